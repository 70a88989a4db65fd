// gfx950 (CDNA4) kernels for C = ReLU(A @ B).
//
// A is (M, K), B is (K, N), C is (M, N), all row-major, one 16-bit dtype
// (fp16 or bf16); products accumulate in fp32 registers, ReLU is applied to the
// fp32 accumulator and the result is rounded to nearest even into the dtype of
// C.  This is the GEMM + ReLU example of "Writing High-Performance Kernels in
// TileLang" (atlascloud.ai, section "Let's write a GEMM"): a block tile of C
// per workgroup, A and B tiles staged through shared memory in a multi-stage
// software pipeline, a tile-level matrix-core product into an fp32 fragment,
// an elementwise max(x, 0) on the fragment, a cast and a store.
//
// Three kernels; the host picks one per call:
//  * gemm_relu_dma, the LDS-DMA kernel (the default for every shape whose rows
//    allow 16- or 4-byte loads): A and B tiles go from L2 into LDS through
//    direct-to-LDS buffer loads in a ring of stages, B stays N-contiguous in
//    LDS and is read K-packed with the gfx950 transpose read.  Its 256 x 256
//    tiles run on 16x16x32 MFMAs, the smaller tiles on 32x32x16.
//  * gemm_relu_tiled, the register-staged kernel, for rows of any length or
//    alignment: loads go through VGPRs, and B is transposed on its way into
//    LDS (two v_perm_b32 per pair of halves), which leaves both LDS tiles
//    K-contiguous.
//  * gemm_relu_direct: one wave per 32x32 block, operands straight from
//    global memory; the fallback, and a structurally different second
//    implementation for the tests.
//
// What changes for CDNA4, in all of them:
//  * The contraction runs on MFMA: v_mfma_f32_32x32x16_{f16,bf16} computes a
//    32x32 fp32 block per instruction, v_mfma_f32_16x16x32 a 16x16 one; both
//    take two 16-byte operand fragments per lane, 8 consecutive k values each
//    (MfmaShape).  At the board's power cap the 16x16x32 form does the same
//    work for less energy, which buys clock.
//  * The MFMA "A" operand is the B^T tile and the "B" operand is the A tile,
//    so the MFMA output block is C^T: each lane then owns 4 consecutive
//    columns of one row of C and stores them with one 8-byte store (or stages
//    them through LDS into whole 128-byte row pieces).
//  * LDS rows of K-contiguous tiles are 128 bytes (BK = 64 halves = 8 chunks
//    of 16 bytes), and their 16-byte chunks are XOR-swizzled per row.  The
//    XOR swizzle is the idea of "TileLang Guide: Composable Tiled AI Kernel
//    Programming" (section "Automated Layout Inference and Bank Conflict
//    Elimination") and of the zwxr.cn hands-on article, section 2.3 (shared
//    memory and bank conflicts); the functions here are chosen for the
//    gfx950 LDS reads each kernel issues (lds_off, a_swizzle, b_swizzle).
//  * Global loads are buffer loads whose descriptor covers only the rows that
//    exist: rows past M (for A) or past K (for B) read as zero in hardware;
//    columns past K (A) or past N (B) are masked by sending the offset out of
//    range.  This is the M/N/K tail handling.
//  * Workgroup ids are remapped so that each of the 8 XCDs (each with its own
//    L2) gets a contiguous range of tiles, and tiles are visited in panels of
//    GROUP_M tile-rows (the rasterization of T.use_swizzle in the pages'
//    listing, re-derived for XCD round-robin dispatch).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Timeline hooks of the LDS-DMA kernel.  They expand to nothing unless a
// measurement program defines GEMM_RELU_TIMELINE before including this header
// (the library never does): then GEMM_RELU_TIMELINE_BEGIN opens a record at
// kernel entry, GEMM_RELU_MARK(p) stamps phase point p (1: the first stage is
// in LDS for every wave; 2: the last unit's K loop is done; 3: its C stores
// are issued) and GEMM_RELU_TIMELINE_END closes the record at exit.
#ifndef GEMM_RELU_TIMELINE
#define GEMM_RELU_TIMELINE_BEGIN
#define GEMM_RELU_MARK(point)
#define GEMM_RELU_TIMELINE_END
#endif

namespace gemm_relu_hip {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

enum Dtype { kF16 = 0, kBF16 = 1 };

// Buffer descriptor word 3 for gfx9-family raw buffers (32-bit data format,
// no swizzle, range checking on).
constexpr int kBufferFlags = 0x00020000;
// An offset that is always beyond every descriptor's num_records: loads from it
// return zero.  The host guarantees num_records < 2^31.
constexpr uint32_t kOobOffset = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}

template <int DT>
__device__ __forceinline__ floatx16 mfma_32x32x16(u32x4 a, u32x4 b, floatx16 c)
{
    if constexpr (DT == kF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a),
                                                      __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// The two MFMA shapes of the LDS-DMA kernel.  Both take 8 consecutive k per
// lane in each operand and retire 1024 flop per SIMD-cycle:
//  32: v_mfma_f32_32x32x16, a 32x32 fp32 block (16 per lane) from 16 k;
//      operand lane l: row l % 32, k 8(l / 32) .. +7.
//  16: v_mfma_f32_16x16x32, a 16x16 fp32 block (4 per lane) from 32 k;
//      operand lane l: row l % 16, k 8(l / 16) .. +7.
// Which 8 k a lane group takes only has to agree between the two operands;
// the LDS-DMA kernel gives 16x16 lane group g = l / 16 the k-block
// kgroup16(g) (see there).
// At the board's power cap the 16x16x32 form sustains more flop per joule: in
// the mfma_form program's MFMA-only loop on N(0, 0.1^2) fp16 register data it
// ran 1971 TFLOP/s at 2040 MHz and 1323 W against 1709 TFLOP/s at 1785 MHz and
// 1300 W for 32x32x16 (0.67 against 0.76 pJ per flop); on zeros, at full
// clock, 723 W against 866 W.
template <int MF>
struct MfmaShape;
template <>
struct MfmaShape<32> {
    using Acc = floatx16;
    static constexpr int KSTEP = 16, ACC = 16;
};
template <>
struct MfmaShape<16> {
    using Acc = floatx4;
    static constexpr int KSTEP = 32, ACC = 4;
};

template <int DT>
__device__ __forceinline__ floatx4 mfma_16x16x32(u32x4 a, u32x4 b, floatx4 c)
{
    if constexpr (DT == kF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, a),
                                                      __builtin_bit_cast(halfx8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// The k-block (8 k of the 32) that lane group g = lane / 16 of a 16x16x32
// operand takes: 0, 2, 1, 3 for g = 0 .. 3, so lanes l and l + 32, which the
// LDS serves together in a 16-byte read, take k-blocks that differ in bit 0
// only, as lanes l and l + 32 do in the 32x32x16 layout (chunks c and c + 1).
// With k-blocks g (0, 1, 2, 3) those lanes read the same rows at chunks c and
// c + 2, which the A-row swizzle puts on the same banks: measured at 8192^3,
// 34.6M bank-conflict cycles per dispatch against 1.0M.
__device__ __forceinline__ int kgroup16(int g)
{
    return ((g & 1) << 1) | (g >> 1);
}

template <int DT, int MF>
__device__ __forceinline__ typename MfmaShape<MF>::Acc mfma(u32x4 a, u32x4 b, typename MfmaShape<MF>::Acc c)
{
    if constexpr (MF == 32)
        return mfma_32x32x16<DT>(a, b, c);
    else
        return mfma_16x16x32<DT>(a, b, c);
}

// ReLU on the fp32 accumulator, then round to nearest even into the dtype.
// x > 0 ? x : 0 (a select, not fmax) so that every x <= 0 gives +0.0.
template <int DT>
__device__ __forceinline__ uint16_t relu_cast(float x)
{
    float r = x > 0.0f ? x : 0.0f;
    if constexpr (DT == kF16)
        return __builtin_bit_cast(uint16_t, (_Float16)r);
    else
        return __builtin_bit_cast(uint16_t, (__bf16)r);
}

// ---------------------------------------------------------------- rasterization

// Map the hardware workgroup id to a (tile_m, tile_n) pair.
//  1. XCD remap: the dispatcher hands workgroup w to XCD w % 8.  Logical id
//     (w % 8) * (T / 8) + w / 8 gives XCD x the contiguous logical range
//     [x * T/8, (x+1) * T/8), so tiles that share A/B panels share one L2.
//     Ids past the last multiple of 8 keep their own number (a bijection).
//  2. Panels: logical ids walk GROUP_M tile-rows at a time, column by column
//     inside the panel, so the tiles in flight reuse the same few A row-panels
//     and B column-panels.
//  xcd_remap = false skips step 1 (the ablation of the remap; results are the
//  same, only which L2 serves which tiles changes).
__device__ __forceinline__ void tile_coords(int wg, int tiles_m, int tiles_n, int group_m,
                                            int& tm, int& tn, bool xcd_remap = true)
{
    const int total = tiles_m * tiles_n;
    const int per_xcd = total / 8;
    int pid = wg;
    if (xcd_remap && wg < per_xcd * 8) pid = (wg % 8) * per_xcd + wg / 8;
    const int panel = group_m * tiles_n;
    const int first_m = (pid / panel) * group_m;
    const int rows = min(tiles_m - first_m, group_m);
    const int in_panel = pid % panel;
    tm = first_m + in_panel % rows;
    tn = in_panel / rows;
}

// ---------------------------------------------------------------- global loads

// Load 8 consecutive 16-bit elements starting at byte offset `off` of the
// buffer, as VEC-element pieces; piece p is read only if valid(p) and is zero
// otherwise.  VEC divides the row length, so a piece is all in or all out.
template <int VEC, class Valid>
__device__ __forceinline__ u32x4 load_chunk(__amdgpu_buffer_rsrc_t rsrc, uint32_t off, Valid valid)
{
    if constexpr (VEC == 8) {
        return __builtin_amdgcn_raw_buffer_load_b128(rsrc, valid(0) ? off : kOobOffset, 0, 0);
    } else if constexpr (VEC == 4) {
        u32x2 lo = __builtin_amdgcn_raw_buffer_load_b64(rsrc, valid(0) ? off : kOobOffset, 0, 0);
        u32x2 hi = __builtin_amdgcn_raw_buffer_load_b64(rsrc, valid(1) ? off + 8 : kOobOffset, 0, 0);
        return u32x4{lo.x, lo.y, hi.x, hi.y};
    } else if constexpr (VEC == 2) {
        u32x4 r;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            r[p] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, valid(p) ? off + 4 * p : kOobOffset, 0, 0);
        return r;
    } else {
        static_assert(VEC == 1, "VEC must be 1, 2, 4 or 8");
        uint32_t h[8];
#pragma unroll
        for (int p = 0; p < 8; ++p)
            h[p] = __builtin_amdgcn_raw_buffer_load_b16(rsrc, valid(p) ? off + 2 * p : kOobOffset, 0, 0);
        return u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    }
}

// ---------------------------------------------------------------- LDS layout

// Byte offset of logical 16-byte chunk c (0..7) of row r in a 128-byte-row tile
// of the register-staged kernel: chunk c of row r sits at chunk position
// c ^ ((r ^ (r >> 3)) & 7).  A ds_read_b128 of 16 consecutive rows at one
// logical chunk lands in 16 distinct 16-byte bank groups (a 256-byte window).
__device__ __forceinline__ uint32_t lds_off(int r, int c)
{
    return (uint32_t)(r * 128 + ((c ^ ((r ^ (r >> 3)) & 7)) << 4));
}

// ---------------------------------------------------------------- epilogue

// Store the ReLU'd fp32 values of one MFMA output block.  `acc` is the 32x32
// block of C^T at (n_base .. n_base+31, m_base .. m_base+31): lane l, register
// 4q + e holds C[m_base + l % 32][n_base + 8q + 4(l / 32) + e].
template <int DT>
__device__ __forceinline__ void store_block(uint16_t* __restrict__ C, const floatx16& acc, int lane,
                                            int m_base, int n_base, int M, int N, bool vec_ok)
{
    const int m = m_base + (lane & 31);
    if (m >= M) return;
    uint16_t* crow = C + (size_t)m * (size_t)N;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int n = n_base + 8 * q + 4 * (lane >> 5);
        uint16_t h0 = relu_cast<DT>(acc[4 * q + 0]);
        uint16_t h1 = relu_cast<DT>(acc[4 * q + 1]);
        uint16_t h2 = relu_cast<DT>(acc[4 * q + 2]);
        uint16_t h3 = relu_cast<DT>(acc[4 * q + 3]);
        if (vec_ok && n + 3 < N) {
            u32x2 v = {(uint32_t)h0 | ((uint32_t)h1 << 16), (uint32_t)h2 | ((uint32_t)h3 << 16)};
            *reinterpret_cast<u32x2*>(crow + n) = v;
        } else {
            if (n + 0 < N) crow[n + 0] = h0;
            if (n + 1 < N) crow[n + 1] = h1;
            if (n + 2 < N) crow[n + 2] = h2;
            if (n + 3 < N) crow[n + 3] = h3;
        }
    }
}

// Store one wave's output, FN x FM blocks as store_block takes them (block
// (i, j) covers rows m_base + 32j .. +31 and columns n_base + 32i .. +31),
// through the wave's 4 KiB LDS strip.  Per round, blocks (2p, j) and (2p+1, j),
// 32 rows x 64 columns, are ReLU'd, rounded and written to the strip; then
// each row piece is read back and stored as 16-byte pieces, 8 lanes per
// 128-byte row piece, instead of 8-byte pieces of 32 different rows.  Strip
// rows are 128 bytes, and 16-byte chunk c of row r sits at chunk
// c ^ ((r >> 1) & 7): the 16-byte reads (16 lanes: 2 rows x 8 chunks) are
// conflict-free.  (The 8-byte writes show 4 bank-conflict cycles each in the
// SQ counters with this layout, with its halves swapped in rows 16-31, and
// as pairs of 4-byte writes spread over all 64 banks alike: measured, and
// the same kernel time.)  A wave's LDS accesses complete in order, so one
// round's reads finish before the next round's writes reuse the strip.
//  The stores are non-temporal buffer stores (cache policy nt): C is written
//  once and never read here, and streaming it keeps the A and B panels in L2
//  when every CU finishes a tile at the same moment (measured: +1.5% at
//  8192^3 over plain stores).  Each round's descriptor covers the valid rows
//  of its 32-row strip (at most 32 * 2^24 * 2 bytes), so rows past M fall
//  outside it and the hardware drops them; pieces past N get an offset past
//  every descriptor.  Needs N % 8 == 0 (a piece is wholly in or out) and a
//  16-byte aligned C.
template <int DT, int FN, int FM>
__device__ __forceinline__ void store_tile_staged(uint16_t* __restrict__ C, const floatx16 (&acc)[FN][FM],
                                                  uint8_t* strip, int lane, int m_base, int n_base, int M, int N)
{
    static_assert(FN % 2 == 0, "pairs of 32-column blocks");
    constexpr int kNonTemporal = 2;   // cache policy nt
    const int rw = lane & 31, h = lane >> 5;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        const int m_strip = m_base + 32 * j;
        const int rows = max(0, min(32, M - m_strip));
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(C + (size_t)max(0, min(m_strip, M)) * (size_t)N,
                                                    (uint32_t)rows * (uint32_t)N * 2u);
#pragma unroll
        for (int p = 0; p < FN / 2; ++p) {
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // lane l, registers 4q .. 4q+3: row l % 32, columns 32ii + 8q + 4(l / 32) + 0..3
                    const floatx16& a = acc[2 * p + ii][j];
                    const uint32_t lo = (uint32_t)relu_cast<DT>(a[4 * q]) | ((uint32_t)relu_cast<DT>(a[4 * q + 1]) << 16);
                    const uint32_t hi =
                        (uint32_t)relu_cast<DT>(a[4 * q + 2]) | ((uint32_t)relu_cast<DT>(a[4 * q + 3]) << 16);
                    *reinterpret_cast<u32x2*>(strip + rw * 128 + (((4 * ii + q) ^ ((rw >> 1) & 7)) << 4) + 8 * h) =
                        u32x2{lo, hi};
                }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int r = 8 * s + (lane >> 3), c = lane & 7;
                const u32x4 v = *reinterpret_cast<const u32x4*>(strip + r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
                const int n = n_base + 64 * p + 8 * c;
                const uint32_t off = n < N ? ((uint32_t)r * (uint32_t)N + (uint32_t)n) * 2u : kOobOffset;
                __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, kNonTemporal);
            }
        }
    }
}

// The same two stores for 16x16 MFMA output blocks.  `acc` is the 16x16 block
// of C^T at (n_base .. +15, m_base .. +15): lane l, register e holds
// C[m_base + l % 16][n_base + 4(l / 16) + e].
template <int DT>
__device__ __forceinline__ void store_block16(uint16_t* __restrict__ C, const floatx4& acc, int lane, int m_base,
                                              int n_base, int M, int N, bool vec_ok)
{
    const int m = m_base + (lane & 15);
    if (m >= M) return;
    uint16_t* crow = C + (size_t)m * (size_t)N;
    const int n = n_base + 4 * (lane >> 4);
    const uint16_t h0 = relu_cast<DT>(acc[0]), h1 = relu_cast<DT>(acc[1]);
    const uint16_t h2 = relu_cast<DT>(acc[2]), h3 = relu_cast<DT>(acc[3]);
    if (vec_ok && n + 3 < N) {
        *reinterpret_cast<u32x2*>(crow + n) =
            u32x2{(uint32_t)h0 | ((uint32_t)h1 << 16), (uint32_t)h2 | ((uint32_t)h3 << 16)};
    } else {
        if (n + 0 < N) crow[n + 0] = h0;
        if (n + 1 < N) crow[n + 1] = h1;
        if (n + 2 < N) crow[n + 2] = h2;
        if (n + 3 < N) crow[n + 3] = h3;
    }
}

// Staged store of FN x FM 16x16 blocks (block (i, j): rows m_base + 16j ..
// +15, columns n_base + 16i .. +15) through the wave's 4 KiB strip: per round,
// the 8 blocks of a 32-row x 64-column piece are written to the strip (lane l
// of block (i, j): strip row 16(j % 2) + l % 16, columns 16(i % 4) + 4(l / 16)
// .. +3), then stored as 16-byte pieces exactly as store_tile_staged does.
// The strip keeps its chunk swizzle c ^ ((r >> 1) & 7); the 8-byte writes
// show 4 bank-conflict cycles each in the SQ counters, as the 32x32 form's do
// (1.0M cycles per 8192^3 launch against 103M LDS-active cycles).
template <int DT, int FN, int FM>
__device__ __forceinline__ void store_tile_staged16(uint16_t* __restrict__ C, const floatx4 (&acc)[FN][FM],
                                                    uint8_t* strip, int lane, int m_base, int n_base, int M, int N)
{
    static_assert(FN % 4 == 0 && FM % 2 == 0, "32-row x 64-column pieces of 16x16 blocks");
    constexpr int kNonTemporal = 2;   // cache policy nt
    const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int jj = 0; jj < FM / 2; ++jj) {
        const int m_strip = m_base + 32 * jj;
        const int rows = max(0, min(32, M - m_strip));
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(C + (size_t)max(0, min(m_strip, M)) * (size_t)N,
                                                    (uint32_t)rows * (uint32_t)N * 2u);
#pragma unroll
        for (int p = 0; p < FN / 4; ++p) {
#pragma unroll
            for (int jh = 0; jh < 2; ++jh)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const floatx4& a = acc[4 * p + ii][2 * jj + jh];
                    const int rw = 16 * jh + r16, c = 2 * ii + (g >> 1);
                    const uint32_t lo = (uint32_t)relu_cast<DT>(a[0]) | ((uint32_t)relu_cast<DT>(a[1]) << 16);
                    const uint32_t hi = (uint32_t)relu_cast<DT>(a[2]) | ((uint32_t)relu_cast<DT>(a[3]) << 16);
                    *reinterpret_cast<u32x2*>(strip + rw * 128 + ((c ^ ((rw >> 1) & 7)) << 4) + 8 * (g & 1)) =
                        u32x2{lo, hi};
                }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int r = 8 * s + (lane >> 3), c = lane & 7;
                const u32x4 v = *reinterpret_cast<const u32x4*>(strip + r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
                const int n = n_base + 64 * p + 8 * c;
                const uint32_t off = n < N ? ((uint32_t)r * (uint32_t)N + (uint32_t)n) * 2u : kOobOffset;
                __builtin_amdgcn_raw_buffer_store_b128(v, rc, off, 0, kNonTemporal);
            }
        }
    }
}

// ---------------------------------------------------------------- tiled kernel

// BM x BN x 64 block tile, WAVES_M x WAVES_N waves, two LDS stages with the
// next tile's global loads in flight (in registers) while the current tile's
// MFMAs run.  VA / VB: elements per global load of A / B (8 needs K % 8 == 0 /
// N % 8 == 0 and 16-byte aligned base pointers; smaller widths need less).
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int GROUP_M_>
struct TileConfig {
    static constexpr int BM = BM_;
    static constexpr int BN = BN_;
    static constexpr int BK = 64;
    static constexpr int WAVES_M = WAVES_M_;
    static constexpr int WAVES_N = WAVES_N_;
    static constexpr int GROUP_M = GROUP_M_;
    static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
    static constexpr int WTM = BM / WAVES_M;          // wave tile rows (m)
    static constexpr int WTN = BN / WAVES_N;          // wave tile cols (n)
    static constexpr int FM = WTM / 32;               // 32x32 MFMA blocks per wave along m
    static constexpr int FN = WTN / 32;               // ... along n
    static constexpr int ROW_BYTES = BK * 2;          // 128
    static constexpr int A_BYTES = BM * ROW_BYTES;
    static constexpr int B_BYTES = BN * ROW_BYTES;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int STAGES = 2;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static constexpr int A_CHUNKS = BM * (BK / 8) / THREADS;    // 16-byte A chunks per thread
    static constexpr int KB = BK * BN / 8 / THREADS;            // B rows per thread (x 8 columns)
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32x32");
    static_assert(A_CHUNKS * THREADS == BM * (BK / 8), "A tile must split evenly over threads");
    static_assert(KB == 8 || KB == 4, "each thread transposes an 8x8 or 4x8 piece of B");
    static_assert(KB * 8 * THREADS == BK * BN, "B tile must split evenly over threads");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one gfx950 CU");
};

// B_NK: B is given as B^T, an (N, K) row-major array.  Its rows are K-contiguous
// like A's, so its tile is loaded and stored exactly as A's (no transpose), and
// the fragment reads are unchanged.  VB then counts elements along K.
template <class Cfg, int DT, int VA, int VB, bool B_NK = false>
__global__ __launch_bounds__(Cfg::THREADS, 1) void gemm_relu_tiled(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C,
    int M, int N, int K, int tiles_m, int tiles_n, int c_vec_ok)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
    constexpr int THREADS = Cfg::THREADS, KB = Cfg::KB;
    __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / Cfg::WAVES_N;
    const int wn = wave % Cfg::WAVES_N;

    int tm, tn;
    tile_coords(blockIdx.x, tiles_m, tiles_n, Cfg::GROUP_M, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;

    // A descriptor: rows m0 .. m0 + valid_m - 1 only; later rows read as zero.
    const int valid_m = min(BM, M - m0);
    const __amdgpu_buffer_rsrc_t rsrc_a =
        make_rsrc(A + (size_t)m0 * (size_t)K, (uint32_t)valid_m * (uint32_t)K * 2u);

    // Per-thread A chunk coordinates (row, logical chunk) inside the tile.
    int a_row[Cfg::A_CHUNKS], a_chunk[Cfg::A_CHUNKS];
#pragma unroll
    for (int i = 0; i < Cfg::A_CHUNKS; ++i) {
        const int q = tid + i * THREADS;
        a_row[i] = q / (BK / 8);
        a_chunk[i] = q % (BK / 8);
    }
    // Per-thread B piece: rows kb*KB .. +KB-1 of the K tile, columns nb*8 .. +7.
    const int b_nb = tid % (BN / 8);
    const int b_kb = tid / (BN / 8);
    const int b_col = n0 + b_nb * 8;
    const uint32_t b_off = (uint32_t)(b_kb * KB) * (uint32_t)N * 2u + (uint32_t)b_col * 2u;
    // B^T (B_NK): rows n0 .. n0 + valid_n - 1 of the (N, K) array; chunks as A's.
    constexpr int BT_CHUNKS = BN * (BK / 8) / THREADS;
    static_assert(!B_NK || BT_CHUNKS * THREADS == BN * (BK / 8), "B^T tile must split evenly over threads");
    const __amdgpu_buffer_rsrc_t rsrc_bt =
        make_rsrc(B + (size_t)(B_NK ? n0 : 0) * (size_t)K, B_NK ? (uint32_t)min(BN, N - n0) * (uint32_t)K * 2u : 0u);

    u32x4 ra[Cfg::A_CHUNKS];
    u32x4 rb[B_NK ? BT_CHUNKS : KB];

    auto global_load = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < Cfg::A_CHUNKS; ++i) {
            const int kc = k0 + a_chunk[i] * 8;
            const uint32_t off = (uint32_t)a_row[i] * (uint32_t)K * 2u + (uint32_t)kc * 2u;
            ra[i] = load_chunk<VA>(rsrc_a, off, [&](int p) { return kc + p * VA < K; });
        }
        if constexpr (B_NK) {
#pragma unroll
            for (int i = 0; i < BT_CHUNKS; ++i) {
                const int q = tid + i * THREADS;
                const int kc = k0 + (q % (BK / 8)) * 8;
                const uint32_t off = (uint32_t)(q / (BK / 8)) * (uint32_t)K * 2u + (uint32_t)kc * 2u;
                rb[i] = load_chunk<VB>(rsrc_bt, off, [&](int p) { return kc + p * VB < K; });
            }
        } else {
            const int valid_k = min(BK, K - k0);
            const __amdgpu_buffer_rsrc_t rsrc_b =
                make_rsrc(B + (size_t)k0 * (size_t)N, (uint32_t)valid_k * (uint32_t)N * 2u);
#pragma unroll
            for (int r = 0; r < KB; ++r)
                rb[r] = load_chunk<VB>(rsrc_b, b_off + (uint32_t)r * (uint32_t)N * 2u,
                                       [&](int p) { return b_col + p * VB < N; });
        }
    };

    auto lds_store = [&](int stage) {
        uint8_t* As = smem + stage * Cfg::STAGE_BYTES;
        uint8_t* Bs = As + Cfg::A_BYTES;
#pragma unroll
        for (int i = 0; i < Cfg::A_CHUNKS; ++i)
            *reinterpret_cast<u32x4*>(As + lds_off(a_row[i], a_chunk[i])) = ra[i];
        if constexpr (B_NK) {
#pragma unroll
            for (int i = 0; i < BT_CHUNKS; ++i) {
                const int q = tid + i * THREADS;
                *reinterpret_cast<u32x4*>(Bs + lds_off(q / (BK / 8), q % (BK / 8))) = rb[i];
            }
        } else {
            // Transpose the KB x 8 piece of B (rows k, 8 columns n) into 8 rows of
            // B^T with KB consecutive k each.  Halves n of row k sit in dword n / 2.
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                const uint32_t sel = (n & 1) ? 0x07060302u : 0x05040100u;
                const int row = b_nb * 8 + n;
                if constexpr (KB == 8) {
                    u32x4 v;
#pragma unroll
                    for (int kp = 0; kp < 4; ++kp)
                        v[kp] = __builtin_amdgcn_perm(rb[2 * kp + 1][n >> 1], rb[2 * kp][n >> 1], sel);
                    *reinterpret_cast<u32x4*>(Bs + lds_off(row, b_kb)) = v;
                } else {
                    u32x2 v;
#pragma unroll
                    for (int kp = 0; kp < 2; ++kp)
                        v[kp] = __builtin_amdgcn_perm(rb[2 * kp + 1][n >> 1], rb[2 * kp][n >> 1], sel);
                    *reinterpret_cast<u32x2*>(Bs + lds_off(row, b_kb >> 1) + (b_kb & 1) * 8) = v;
                }
            }
        }
    };

    floatx16 acc[Cfg::FN][Cfg::FM];
#pragma unroll
    for (int i = 0; i < Cfg::FN; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FM; ++j)
            acc[i][j] = floatx16{0};

    const int KT = (K + BK - 1) / BK;
    const int frag_row = lane & 31;
    const int frag_chunk = lane >> 5;

    if (KT > 0) {
        global_load(0);
        lds_store(0);
        __syncthreads();
    }
    for (int kt = 0; kt < KT; ++kt) {
        const int stage = kt & 1;
        if (kt + 1 < KT) global_load(kt + 1);

        const uint8_t* As = smem + stage * Cfg::STAGE_BYTES;
        const uint8_t* Bs = As + Cfg::A_BYTES;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int chunk = ks * 2 + frag_chunk;
            u32x4 fa[Cfg::FN], fb[Cfg::FM];
#pragma unroll
            for (int i = 0; i < Cfg::FN; ++i)
                fa[i] = *reinterpret_cast<const u32x4*>(Bs + lds_off(wn * Cfg::WTN + i * 32 + frag_row, chunk));
#pragma unroll
            for (int j = 0; j < Cfg::FM; ++j)
                fb[j] = *reinterpret_cast<const u32x4*>(As + lds_off(wm * Cfg::WTM + j * 32 + frag_row, chunk));
#pragma unroll
            for (int i = 0; i < Cfg::FN; ++i)
#pragma unroll
                for (int j = 0; j < Cfg::FM; ++j)
                    acc[i][j] = mfma_32x32x16<DT>(fa[i], fb[j], acc[i][j]);
        }

        if (kt + 1 < KT) lds_store(stage ^ 1);
        __syncthreads();
    }

    // Fused epilogue: ReLU, round to the dtype, masked store.
#pragma unroll
    for (int i = 0; i < Cfg::FN; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::FM; ++j)
            store_block<DT>(C, acc[i][j], lane, m0 + wm * Cfg::WTM + j * 32, n0 + wn * Cfg::WTN + i * 32,
                            M, N, c_vec_ok != 0);
}

// ---------------------------------------------------------------- LDS-DMA kernel

// Block tile BM x BN x BK, a ring of STAGES LDS stages filled by direct-to-LDS
// buffer loads (buffer_load_dwordx4 ... lds): tile data goes from L2 into LDS
// without passing through VGPRs, so loads run STAGES-1 K-steps ahead of the
// MFMAs at no register cost.  This is the pages' multi-stage software
// pipeline (T.Pipelined with several stages in flight), built from gfx950 LDS
// DMA instead of cp.async/TMA.  The large instance (256x256x64, 2 stages)
// runs 8 waves of 128x64 on 16x16x32 MFMAs, two per SIMD, so one wave's LDS
// and barrier waits are covered by the other's MFMAs; the small instance
// (64x64x64, 8 stages) keeps 7 stages of loads in flight for latency- and
// HBM-bound shapes.
//
// LDS layout: all A stages first, then all B stages.
//  * A stage: BM rows (m) x BK k, K-contiguous as in memory, rows of BK*2
//    bytes, 16-byte chunks swizzled by a_swizzle (conflict-free
//    ds_read_b128 of 16 consecutive rows).
//  * B stage: BK rows (k) x BN n, kept N-contiguous as it is in memory, rows
//    of BN*2 bytes, chunks swizzled by b_swizzle.  MFMA operands need 8
//    consecutive k per lane; ds_read_b64_tr_b16 gives them 4 at a time:
//    within each group of 16 lanes, source lane s points at row s / 4,
//    columns 4 (s % 4) .. +3 of a 4 x 16 block, and lane j receives the 4 k
//    values of column j.
// A DMA instruction writes 1 KB of LDS at consecutive 16-byte slots (lane l at
// base + 16 l); the swizzle is applied by choosing which global chunk lane l
// fetches.
//
// One K-step is BK/KSTEP MFMA k-steps (KSTEP = 16 or 32 k); the work of each
// (the next k-step's fragment reads and, in the first, the DMA of stage
// kt+STAGES-1; with early refill, in the last, that of stage kt+STAGES) is
// spread one group per MFMA.  In the last k-step the wave waits for stage
// kt+1 and meets the other waves at the barrier, then reads stage kt+1's
// first fragments while the last MFMAs of stage kt run.  The loop body has no
// branches: stages past the end are "loaded" through a zero-length buffer
// descriptor (nothing is fetched).
//
// Synchronisation: the DMA loads are issued from inline assembly, so the
// compiler does not add its own (maximal) waits before LDS reads; the kernel
// waits for exactly the loads of the stage it is about to read
// (s_waitcnt vmcnt) before the barrier.
//
// The workgroups are persistent (one per CU): each computes every G-th tile
// and streams the K-steps of all its tiles through one ring, so a tile's
// first stages are already in LDS when the previous tile's epilogue runs, and
// no workgroup is dispatched, started or drained between tiles.

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef int int32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor as four dwords (base, stride 0, num_records, flags).
__device__ __forceinline__ int32x4_t rsrc_words(const void* base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return int32x4_t{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, kBufferFlags};
}

// 64 lanes x 16 bytes from the buffer into LDS [lds_addr, lds_addr + 1024).
// voffset is per lane, soffset is uniform.
__device__ __forceinline__ void dma_b128(int32x4_t rsrc, uint32_t lds_addr, uint32_t voffset, uint32_t soffset)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds_addr), "v"(voffset), "s"(rsrc), "s"(soffset)
                 : "memory", "m0");
}

// 64 lanes x 4 bytes from the buffer into LDS [lds_addr, lds_addr + 256).
__device__ __forceinline__ void dma_b32(int32x4_t rsrc, uint32_t lds_addr, uint32_t voffset, uint32_t soffset)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :
                 : "s"(lds_addr), "v"(voffset), "s"(rsrc), "s"(soffset)
                 : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// All of this wave's LDS reads are complete, then the workgroup barrier.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

__device__ __forceinline__ u32x2 ds_read_tr16(const uint8_t* p)
{
    short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) short4_t*)(p));
    return __builtin_bit_cast(u32x2, v);
}

// Swizzle of the 16-byte chunks of one K-contiguous A row of ROW bytes (64 or
// 128): chunk c of row r is stored at chunk c ^ a_swizzle(r).  Sixteen lanes
// that read 16 consecutive rows at one logical chunk (one ds_read_b128 issue
// group) land in 16 distinct 16-byte bank groups, and the function is
// unchanged by adding a multiple of 16 rows.
template <int ROW>
__device__ __forceinline__ int a_swizzle(int r)
{
    static_assert(ROW == 64 || ROW == 128, "A rows of 32 or 64 k");
    if constexpr (ROW == 64)
        return (r >> 2) & 3;             // 4 rows share a 256-byte bank window
    else
        return (r ^ ((r >> 3) & 1)) & 7; // 2 rows share a 256-byte bank window
}

// Swizzle of the 16-byte chunks of one N-contiguous B row of ROW bytes (64,
// 128, 256 or 512).  A ds_read_b64_tr_b16 pair of 16-lane groups reads 4
// consecutive rows (k % 4 == 0) x 4 consecutive chunks (32 columns); the XOR
// term spreads those 16 chunks over 16 distinct bank groups.  It depends on k
// only through bits the fragment offsets (multiples of 4 rows) leave alone.
// Rows of 64 bytes need none: 4 of them fill one 256-byte bank window.
//  With 16x16 MFMAs (MF = 16) the two 16-lane groups of a pair read rows k and
//  k + 16 (4 rows each, k-blocks kgroup16(0) and kgroup16(1)) x 2 chunks (16
//  columns); the extra term 2 * (bit 4 of k) moves the second group's chunks
//  off the first's.
template <int ROW, int MF = 32>
__device__ __forceinline__ int b_swizzle(int k)
{
    static_assert(ROW == 64 || ROW == 128 || ROW == 256 || ROW == 512, "B rows of 32, 64, 128 or 256 n");
    const int k16 = MF == 16 ? 2 * ((k >> 4) & 1) : 0;
    if constexpr (ROW == 64)
        return k16;
    else if constexpr (ROW == 128)
        return 4 * ((k >> 1) & 1) ^ k16;  // 2 rows share a 256-byte bank window
    else
        return 4 * (k & 3) ^ k16;         // every row starts at bank 0
}

template <int BM_, int BN_, int BK_, int STAGES_, int WAVES_M_, int WAVES_N_, int GROUP_M_,
          int A_LANE_BYTES_ = 16, int B_LANE_BYTES_ = 16, bool B_KMAJOR_ = false, int PRODUCERS_ = 0,
          bool SWIZZLE_ = true, bool XCD_REMAP_ = true, int MFMA_ = 32, bool EARLY_REFILL_ = false,
          bool K_ROTATE_ = false>
struct DmaConfig {
    // SWIZZLE = false stores every LDS row unpermuted (the ablation of the XOR
    // swizzle; results are the same, only the bank conflicts differ).
    // XCD_REMAP = false maps tiles to workgroups without the XCD remap (the
    // ablation of the remap; results are the same).
    static constexpr bool SWIZZLE = SWIZZLE_, XCD_REMAP = XCD_REMAP_;
    static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_, GROUP_M = GROUP_M_;
    // WAVES compute waves; PRODUCERS > 0 adds that many waves that only issue
    // the LDS DMA (wave specialisation), else every compute wave loads its share.
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, WAVES = WAVES_M * WAVES_N;
    static constexpr int PRODUCERS = PRODUCERS_, DMA_WAVES = PRODUCERS > 0 ? PRODUCERS : WAVES;
    static constexpr int THREADS = 64 * (WAVES + PRODUCERS);
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;     // wave tile
    // MFMA shape (MfmaShape): 32 (32x32x16) or 16 (16x16x32).
    static constexpr int MF = MFMA_, KSTEP = MfmaShape<MF>::KSTEP;
    using Acc = typename MfmaShape<MF>::Acc;
    static constexpr int FM = WTM / MF, FN = WTN / MF;               // MFMA blocks per wave
    static constexpr int NKS = BK / KSTEP;                           // MFMA k-steps per stage
    // EARLY_REFILL: a ring slot is refilled as soon as the step barrier frees
    // it, in the last k-step of the step that read it, instead of in the first
    // k-step of the next step (see the main loop).
    static constexpr bool EARLY_REFILL = EARLY_REFILL_;
    // B_KMAJOR: B is given as B^T, an (N, K) row-major array, so its LDS stage
    // has A's shape (BN rows of BK k) and its fragments are plain ds_read_b128.
    static constexpr bool B_KMAJOR = B_KMAJOR_;
    // K_ROTATE (B stored (N, K) only): with at most 64 rows of A, each tile
    // walks its K-steps from a start set by its column, wrapping round, instead
    // of from 0 (see the load side of the kernel).
    static constexpr bool K_ROTATE = K_ROTATE_;
    static_assert(!K_ROTATE || B_KMAJOR_, "K rotation is for B stored (N, K)");
    static constexpr int A_ROW = BK * 2, B_ROW = B_KMAJOR ? BK * 2 : BN * 2;   // bytes per LDS row
    static constexpr int A_STAGE = BM * A_ROW, B_STAGE = BN * BK * 2;          // bytes per stage
    static constexpr int B_REGION = STAGES * A_STAGE;                // B stages follow the A stages
    static constexpr int LDS_BYTES = STAGES * (A_STAGE + B_STAGE);
    // C staging: each compute wave writes its finished output through a
    // private 4 KiB LDS strip past the ring (32 rows x 64 columns at a time),
    // so that C leaves as whole 128-byte row pieces.  Needs a wave tile of
    // whole 32 x 64 pieces and room in the 160 KiB; else 0 and C is stored
    // straight from the accumulators.
    static constexpr int C_STAGE_WAVE =
        (WTN % 64 == 0 && WTM % 32 == 0 && LDS_BYTES + WAVES * 4096 <= 160 * 1024) ? 4096 : 0;
    static constexpr int C_STAGE_BYTES = WAVES * C_STAGE_WAVE;
    // Bytes each lane moves per DMA instruction: 16 (buffer_load_dwordx4, needs
    // rows of a multiple of 8 elements) or 4 (buffer_load_dword, rows of an even
    // number of elements).
    static constexpr int A_LANE_BYTES = A_LANE_BYTES_, B_LANE_BYTES = B_LANE_BYTES_;
    static constexpr int QA = A_STAGE / (64 * A_LANE_BYTES) / DMA_WAVES; // DMA instructions per wave per stage
    static constexpr int QB = B_STAGE / (64 * B_LANE_BYTES) / DMA_WAVES;
    static constexpr int NQ = QA + QB;
    static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile of whole MFMA blocks");
    static_assert(BK % (2 * KSTEP) == 0, "an even number of MFMA k-steps per stage");
    static_assert((A_LANE_BYTES == 16 || A_LANE_BYTES == 4) && (B_LANE_BYTES == 16 || B_LANE_BYTES == 4),
                  "dwordx4 or dword DMA");
    static_assert(QA * DMA_WAVES * 64 * A_LANE_BYTES == A_STAGE && QB * DMA_WAVES * 64 * B_LANE_BYTES == B_STAGE,
                  "stages split evenly into DMA instructions");
    static_assert((STAGES & (STAGES - 1)) == 0 && STAGES >= 2, "power-of-two ring of at least 2 stages");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one gfx950 CU");
    static_assert((STAGES - 2) * NQ < 64, "vmcnt range");
};

// The LDS-DMA kernel: block tile BM x BN x BK, a ring of STAGES LDS stages
// filled by direct-to-LDS loads, WAVES_M x WAVES_N waves of MF x MF MFMA blocks.
// KTAIL 0: K is a multiple of BK.  KTAIL 1: it is not, so the last stage is
// partial and its A pieces past K are masked (K must still be a multiple of
// the piece: 8 elements for 16-byte lanes, 2 for 4-byte lanes).  KTAIL 2: as
// 1, with 16-byte lanes for K-contiguous rows (A, and B^T when B is stored
// (N, K)) of any even K (rows 4-byte aligned).  When K % 8 is not 0, the piece
// holding element K - 1 of such a row also holds elements past K, which its
// DMA takes from the next row (or reads as zero past the descriptor).  Once
// the last stage of a tile has landed, every thread rewrites half of one row's
// such piece in LDS from two exact 4-byte loads (zero past K), for A and B^T,
// and one extra barrier orders those writes before the fragment reads.
// KTAIL 2 needs a 2-stage ring, no producer waves and two threads per row.
// SPLITK: each tile's K range is cut into `splits` contiguous parts, each a
// work unit of its own (for shapes with fewer tiles than CUs).  When a unit
// finishes, each of its waves writes its fp32 partial sub-tile to `ws` and
// counts itself in `counters[tile * WAVES + wave]`; the wave that finds all
// other parts counted adds their partials in part order (so the result does
// not depend on which part finishes last), applies ReLU, stores C and resets
// the counter to zero.  Nothing ever waits for another wave or workgroup.
// Without SPLITK, `ws`, `counters` and `splits` are unused.
template <class Cfg, int DT, int KTAIL, bool SPLITK = false>
__global__ __launch_bounds__(Cfg::THREADS, 1) void gemm_relu_dma(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C,
    int M, int N, int K, int tiles_m, int tiles_n, int c_vec_ok,
    float* __restrict__ ws, int* __restrict__ counters, int splits_arg)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, S = Cfg::STAGES;
    constexpr int QA = Cfg::QA, QB = Cfg::QB, NQ = Cfg::NQ, FM = Cfg::FM, FN = Cfg::FN;
    constexpr int WTM = Cfg::WTM, WTN = Cfg::WTN, NKS = Cfg::NKS;
    constexpr int A_ROW = Cfg::A_ROW, B_ROW = Cfg::B_ROW;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[Cfg::LDS_BYTES + Cfg::C_STAGE_BYTES];
    GEMM_RELU_TIMELINE_BEGIN

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
    // With producer waves, waves WAVES .. WAVES + PRODUCERS - 1 issue every DMA
    // and compute nothing; dwave is a wave's index among the loading waves.
    constexpr bool WS = Cfg::PRODUCERS > 0;
    const bool producer = WS && wave >= Cfg::WAVES;
    const int dwave = WS ? wave - Cfg::WAVES : wave;

    // Persistent workgroups: workgroup b computes work units b, b + G, b + 2G,
    // ... (G = gridDim.x, a multiple of 8 or all units), and all K-steps of all
    // its units form one stream through the LDS ring, so the first stages of
    // the next unit are loaded while the current one finishes.  A unit is a
    // tile, or with SPLITK one of its `splits` K ranges (unit u: tile u /
    // splits, part u % splits, K-steps [part * KT / splits, (part + 1) * KT /
    // splits)).
    const int splits = SPLITK ? splits_arg : 1;
    const int total_units = tiles_m * tiles_n * splits;
    const int n_units = (total_units - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const int KT = (K + BK - 1) / BK;
    auto unit_info = [&](int i, int& tile, int& part, int& kt0, int& kt1) {
        const int u = (int)blockIdx.x + i * (int)gridDim.x;
        tile = u / splits;
        part = u - tile * splits;
        kt0 = part * KT / splits;
        kt1 = (part + 1) * KT / splits;
    };
    int steps = n_units * KT;
    if constexpr (SPLITK) {
        steps = 0;
        for (int i = 0; i < n_units; ++i) {
            int t, pt, k0, k1;
            unit_info(i, t, pt, k0, k1);
            steps += k1 - k0;
        }
    }
    auto tile_origin = [&](int tile, int& m0, int& n0) {
        int tm, tn;
        tile_coords(tile, tiles_m, tiles_n, Cfg::GROUP_M, tm, tn, Cfg::XCD_REMAP);
        m0 = tm * BM;
        n0 = tn * BN;
    };

    const int32x4_t rsrc_none = rsrc_words(A, 0u);
    const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)smem);

    // DMA source offsets, relative to the tile origin.  A DMA instruction writes
    // 64 * LANE_BYTES consecutive LDS bytes, lane l at byte l * LANE_BYTES; that
    // byte lies in some row and physical 16-byte chunk of the stage, and the
    // lane fetches the logical chunk (and the same bytes inside it) that the
    // swizzle puts there.
    constexpr int LA = Cfg::A_LANE_BYTES, LB = Cfg::B_LANE_BYTES;
    uint32_t a_voff[QA], b_voff[QB];
    int a_kcol[QA], b_ncol[QB];
#pragma unroll
    for (int q = 0; q < QA; ++q) {
        const int byte = ((dwave * QA + q) * 64 + lane) * LA;      // offset inside the A stage
        const int row = byte / A_ROW;
        const int lc = ((byte % A_ROW) / 16) ^ (Cfg::SWIZZLE ? a_swizzle<A_ROW>(row) : 0);
        const int kcol = lc * 8 + (byte % 16) / 2;                  // first k of this lane's piece
        a_voff[q] = (uint32_t)row * (uint32_t)K * 2u + (uint32_t)kcol * 2u;
        a_kcol[q] = kcol;
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
        const int byte = ((dwave * QB + q) * 64 + lane) * LB;      // offset inside the B stage
        const int row = byte / B_ROW;
        if constexpr (Cfg::B_KMAJOR) {                              // row = n, K-contiguous like A
            const int lc = ((byte % B_ROW) / 16) ^ (Cfg::SWIZZLE ? a_swizzle<B_ROW>(row) : 0);
            const int kcol = lc * 8 + (byte % 16) / 2;
            b_voff[q] = (uint32_t)row * (uint32_t)K * 2u + (uint32_t)kcol * 2u;
            b_ncol[q] = kcol;                                       // here: first k of the piece
        } else {                                                    // row = k, N-contiguous
            const int lc = ((byte % B_ROW) / 16) ^ (Cfg::SWIZZLE ? b_swizzle<B_ROW, Cfg::MF>(row) : 0);
            const int ncol = lc * 8 + (byte % 16) / 2;              // first n of this lane's piece, from n0
            b_voff[q] = (uint32_t)row * (uint32_t)N * 2u + (uint32_t)ncol * 2u;
            b_ncol[q] = ncol;
        }
    }
    const uint32_t b_stage_bytes = (uint32_t)BK * (uint32_t)N * 2u;

    // The load side of the stream: the unit and K-step the next DMA belongs to.
    // Past the end of the stream the descriptors are zero-length (f_b_bytes =
    // 0 for B stored (K, N)), so the remaining ring steps fetch nothing
    // without a per-instruction test.
    int f_unit = 0, f_kt = 0, f_kt_end = 0, f_m0 = 0, f_n0 = 0;
    // K rotation.  With B stored (N, K) every tile reads BK elements of each of
    // its B^T rows per K-step; if all tiles take their K-steps in the same
    // order, the whole chip reads the same narrow column of all N rows at once,
    // which streams about 30% slower than spreading the tiles over K (a 128-byte
    // column of 16384 rows of 16 KiB: 4.6 against 6.0 TB/s in a DMA-only
    // pattern).  So, when A has at most 64 rows (it then stays in L2 whatever
    // the order), tile column tn starts at K-step (37 tn) mod KT and wraps
    // round; tiles of one column keep one order and still share B^T in L2.
    // The order changes only how the fp32 sums are grouped.
    constexpr bool KROT = Cfg::K_ROTATE && !SPLITK && KTAIL != 2;
    const bool rotate = KROT && M <= 64;
    int f_k0 = 0;   // with KROT: first k of the step being filled
    int32x4_t f_rsrc_a = rsrc_none, f_rsrc_bt = rsrc_none;
    const uint16_t* f_b_ptr = B;   // B stored (K, N): element (k0, f_n0) of the current step
    uint32_t f_b_bytes = 0;        // ... and the bytes its descriptor covers (a whole stage)
    auto fill_tile_setup = [&]() {
        if (f_unit < n_units) {
            int tile, part;
            unit_info(f_unit, tile, part, f_kt, f_kt_end);
            tile_origin(tile, f_m0, f_n0);
            // rows f_m0 .. f_m0 + valid_m - 1 of A; rows past M read as zero
            const int valid_m = min(BM, M - f_m0);
            f_rsrc_a = rsrc_words(A + (size_t)f_m0 * (size_t)K, (uint32_t)valid_m * (uint32_t)K * 2u);
            if constexpr (Cfg::B_KMAJOR) {   // rows f_n0 .. of B^T; rows past N read as zero
                const int valid_n = min(BN, N - f_n0);
                f_rsrc_bt = rsrc_words(B + (size_t)f_n0 * (size_t)K, (uint32_t)valid_n * (uint32_t)K * 2u);
            } else {
                f_b_ptr = B + (size_t)f_kt * BK * (size_t)N + f_n0;
                f_b_bytes = b_stage_bytes;
            }
        } else {
            f_rsrc_a = f_rsrc_bt = rsrc_none;
            f_b_bytes = 0u;
        }
        // The tile's first K-step to fill (set on every path: a store in one
        // branch only would keep f_k0 out of registers).  Uniform;
        // readfirstlane keeps it in a scalar register.
        if constexpr (KROT) f_k0 = __builtin_amdgcn_readfirstlane((rotate ? (f_n0 / BN * 37) % KT : f_kt) * BK);
    };
    fill_tile_setup();

    auto dma_issue = [&](int32x4_t rsrc, uint32_t lds, uint32_t vo, uint32_t so, int lane_bytes) {
        if (lane_bytes == 16) dma_b128(rsrc, lds, vo, so);
        else dma_b32(rsrc, lds, vo, so);
    };
    // DMA q (0 .. QA-1: A, QA .. NQ-1: B) of the current fill step into ring
    // slot `slot`.  Steps past the end of the stream use a zero-length
    // descriptor: nothing is fetched.
    auto dma = [&](int slot, int q) {
        const int k0 = KROT ? f_k0 : f_kt * BK;
        if (q < QA) {
            uint32_t vo = a_voff[q], so = (uint32_t)k0 * 2u;
            if (KTAIL) {   // pieces that start past K read as zero
                vo = k0 + a_kcol[q] < K ? a_voff[q] + so : kOobOffset;
                so = 0u;
            }
            dma_issue(f_rsrc_a, lds_base + slot * Cfg::A_STAGE + (dwave * QA + q) * 64 * LA, vo, so, LA);
        } else if constexpr (Cfg::B_KMAJOR) {
            const int qb = q - QA;
            uint32_t vo = b_voff[qb], so = (uint32_t)k0 * 2u;
            if (KTAIL) {
                vo = k0 + b_ncol[qb] < K ? b_voff[qb] + so : kOobOffset;
                so = 0u;
            }
            dma_issue(f_rsrc_bt, lds_base + Cfg::B_REGION + slot * Cfg::B_STAGE + (dwave * QB + qb) * 64 * LB, vo, so,
                      LB);
        } else {
            // descriptor based at (row k0, column f_n0): rows past K read as zero
            const uint32_t nb =
                KTAIL ? (f_b_bytes ? (uint32_t)min(BK, K - k0) * (uint32_t)N * 2u : 0u) : f_b_bytes;
            const int32x4_t rb = rsrc_words(f_b_ptr, nb);
            const uint32_t vo = f_n0 + b_ncol[q - QA] < N ? b_voff[q - QA] : kOobOffset;   // columns past N
            dma_issue(rb, lds_base + Cfg::B_REGION + slot * Cfg::B_STAGE + (dwave * QB + (q - QA)) * 64 * LB, vo, 0u,
                      LB);
        }
    };
    auto fill_advance = [&]() {
        if (++f_kt == f_kt_end) {
            ++f_unit;
            fill_tile_setup();
        } else if constexpr (!Cfg::B_KMAJOR) {
            f_b_ptr += (size_t)BK * (size_t)N;
        } else if constexpr (KROT) {
            f_k0 += BK;
            if (f_k0 >= KT * BK) f_k0 = 0;   // wrap round (only when rotating)
        }
    };

    // KTAIL 2: thread t owns dwords 2(t & 1) and 2(t & 1) + 1 of the last
    // K-step's piece holding element K - 1 in row t / 2 of the tile's A rows
    // (and of its B^T rows when B is stored (N, K)).  fix_issue loads them, for
    // the tile at (m0, n0), when that stage is filled (rows past M or N and
    // dwords past K read as zero); fix_apply writes them over what the DMA put
    // there, once the stage has landed for every wave.  A and B^T rows have the
    // same length and swizzle.
    static_assert(KTAIL != 2 || (S == 2 && !WS && LA == 16 && Cfg::THREADS == 2 * BM &&
                                 (!Cfg::B_KMAJOR || (LB == 16 && Cfg::THREADS == 2 * BN && B_ROW == A_ROW))),
                  "KTAIL 2 layout");
    constexpr bool KFIX = KTAIL == 2;
    const int fx_row = threadIdx.x >> 1;
    const int fx_k = (KT - 1) * BK + 8 * (((K - 1) % BK) / 8) + 4 * (threadIdx.x & 1);   // first k of the two dwords
    const uint32_t fx_lds = (uint32_t)(fx_row * A_ROW +
                                       16 * ((((K - 1) % BK) / 8) ^ (Cfg::SWIZZLE ? a_swizzle<A_ROW>(fx_row) : 0)) +
                                       8 * (threadIdx.x & 1));
    u32x2 fx_a = {0u, 0u}, fx_b = {0u, 0u};
    auto fix_load = [&](const uint16_t* rows, int valid_rows) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(rows, (uint32_t)valid_rows * (uint32_t)K * 2u);
        const uint32_t off = (uint32_t)fx_row * (uint32_t)K * 2u + (uint32_t)fx_k * 2u;
        return u32x2{__builtin_amdgcn_raw_buffer_load_b32(rs, fx_k < K ? off : kOobOffset, 0, 0),
                     __builtin_amdgcn_raw_buffer_load_b32(rs, fx_k + 2 < K ? off + 4u : kOobOffset, 0, 0)};
    };
    auto fix_issue = [&](int m0, int n0) {
        fx_a = fix_load(A + (size_t)m0 * (size_t)K, min(BM, M - m0));
        if constexpr (Cfg::B_KMAJOR) fx_b = fix_load(B + (size_t)n0 * (size_t)K, min(BN, N - n0));
    };
    auto fix_apply = [&](int slot) {
        *reinterpret_cast<u32x2*>(smem + slot * Cfg::A_STAGE + fx_lds) = fx_a;
        if constexpr (Cfg::B_KMAJOR)
            *reinterpret_cast<u32x2*>(smem + Cfg::B_REGION + slot * Cfg::B_STAGE + fx_lds) = fx_b;
        lds_barrier();
    };
    // Whether the stage the load side fills next is a tile's last K-step.
    auto fill_is_last_kstep = [&]() { return KFIX && f_unit < n_units && f_kt == KT - 1; };

    // Per-lane LDS read offsets inside a stage (MF = 32 / 16: the MFMA shape;
    // KSTEP = 16 / 32 k per MFMA).  A lane's k-block inside a k-step is kb:
    // lane / 32 for MF = 32, kgroup16(lane / 16) for MF = 16.
    //  A fragment j, k-step ks: row wm*WTM + MF*j + lane%MF, chunk (KSTEP/8)ks + kb.
    constexpr int MF = Cfg::MF, KSTEP = Cfg::KSTEP;
    using Acc = typename Cfg::Acc;
    const int kb = MF == 32 ? lane >> 5 : kgroup16(lane >> 4);
    uint32_t a_frag_off[NKS];
    {
        const int row = wm * WTM + lane % MF;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            a_frag_off[ks] = (uint32_t)(row * A_ROW + 16 * (((KSTEP / 8) * ks + kb) ^
                                                             (Cfg::SWIZZLE ? a_swizzle<A_ROW>(row) : 0)));
    }
    //  B^T fragment i, k-step ks, half hh: lane group g = lane/16, j = lane%16;
    //  MF = 32: row k = 16ks + 8(g/2) + 4hh + j/4, column n = wn*WTN + 32i + 16(g%2) + 4(j%4);
    //  MF = 16: row k = 32ks + 8kgroup16(g) + 4hh + j/4, column n = wn*WTN + 16i + 4(j%4).
    //  (B_KMAJOR: like A, row n = wn*WTN + MF*i + lane%MF, chunk (KSTEP/8)ks + kb.)
    uint32_t b_frag_off[Cfg::B_KMAJOR ? NKS : FN];
    if constexpr (Cfg::B_KMAJOR) {
        const int row = wn * WTN + lane % MF;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            b_frag_off[ks] = (uint32_t)(Cfg::B_REGION + row * B_ROW +
                                        16 * (((KSTEP / 8) * ks + kb) ^ (Cfg::SWIZZLE ? a_swizzle<B_ROW>(row) : 0)));
    } else {
        const int g = lane >> 4, j = lane & 15;
        // + KSTEP*ks + 4hh leave the swizzle unchanged
        const int krow = 8 * (MF == 32 ? g >> 1 : kgroup16(g)) + (j >> 2);
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const int n = wn * WTN + i * MF + (MF == 32 ? 16 * (g & 1) : 0) + 4 * (j & 3);
            b_frag_off[i] = (uint32_t)(Cfg::B_REGION + krow * B_ROW +
                                       16 * ((n >> 3) ^ (Cfg::SWIZZLE ? b_swizzle<B_ROW, MF>(krow) : 0)) +
                                       8 * (j & 1));
        }
    }

    Acc acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = Acc{0};

    // [buffer][fragment]: B^T fragments (MFMA A operand) and A fragments (MFMA B operand)
    u32x4 fa[2][FN], fb[2][FM];
    auto read_a = [&](int buf, int slot, int ks, int j) {
        fb[buf][j] = *reinterpret_cast<const u32x4*>(smem + slot * Cfg::A_STAGE + a_frag_off[ks] + j * MF * A_ROW);
    };
    auto read_b = [&](int buf, int slot, int ks, int i) {
        if constexpr (Cfg::B_KMAJOR) {
            fa[buf][i] = *reinterpret_cast<const u32x4*>(smem + slot * Cfg::B_STAGE + b_frag_off[ks] + i * MF * B_ROW);
        } else {
            const uint8_t* p = smem + slot * Cfg::B_STAGE + b_frag_off[i] + KSTEP * ks * B_ROW;
            const u32x2 lo = ds_read_tr16(p);
            const u32x2 hi = ds_read_tr16(p + 4 * B_ROW);
            fa[buf][i] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
    };
    auto read_unit = [&](int buf, int slot, int ks, int u) {
        if (u < FM) read_a(buf, slot, ks, u);
        else read_b(buf, slot, ks, u - FM);
    };
    constexpr int NF = FM + FN, NMF = FM * FN;

    // The compute side of the stream: the unit being accumulated.
    int c_unit = 0, c_tile, c_part, c_kt, c_kt_end, c_m0, c_n0;
    unit_info(0, c_tile, c_part, c_kt, c_kt_end);
    tile_origin(c_tile, c_m0, c_n0);

    // SPLITK: combine the parts of tile c_tile, wave by wave: wave w of every
    // part owns the same sub-tile, and counts itself in counters[tile * WAVES
    // + w].  The wave that finds the other parts counted holds the last part:
    // it adds theirs and returns true (it stores that sub-tile).  Waves never
    // wait for each other or for other workgroups.
    //  The parts of a tile run on different XCDs, whose L2s are not coherent
    //  with each other.  Partials are therefore written and read with
    //  device-scope (sc1) buffer accesses, coherent without any L2 write-back
    //  or invalidate, and a wave's partial stores have completed (vmcnt 0)
    //  before it counts itself.
    //  Partial layout: tile t, part p, wave w, block (i, j), quarter q, lane l:
    //  4 floats at ((((t * splits + p) * WAVES + w) * FN + i) * FM + j) * 64 ACC
    //  + q * 256 + l * 4 (ACC fp32 per lane per block: 16 or 4), so each
    //  quarter of a block is one contiguous 1 KiB.
    auto combine_parts = [&](Acc (&sum)[FN][FM]) -> bool {
        constexpr int ACC = MfmaShape<MF>::ACC, BLOCK_BYTES = 256 * ACC;   // QUARTERS 1 KiB pieces
        constexpr int QUARTERS = ACC / 4;
        constexpr int kDeviceScope = 16;   // cache policy sc1: coherent at device scope
        const uint32_t tile_bytes = (uint32_t)Cfg::BM * (uint32_t)Cfg::BN * 4u;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(ws + (size_t)c_tile * (size_t)splits * (tile_bytes / 4),
                                                    (uint32_t)splits * tile_bytes);
        auto part_off = [&](int part, int i, int j) {
            return (uint32_t)part * tile_bytes + (uint32_t)((wave * FN + i) * FM + j) * BLOCK_BYTES + lane * 16;
        };
        int* const cnt = counters + (size_t)c_tile * Cfg::WAVES + wave;
        // If every other part has already counted itself, this one is last
        // and need not publish its own partial.
        int seen = 0;
        if (lane == 0) seen = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        bool last = __builtin_amdgcn_readfirstlane(seen) == splits - 1;
        if (!last) {
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j)
#pragma unroll
                    for (int q = 0; q < QUARTERS; ++q) {
                        const floatx4 v = {sum[i][j][4 * q], sum[i][j][4 * q + 1], sum[i][j][4 * q + 2],
                                           sum[i][j][4 * q + 3]};
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs,
                                                               part_off(c_part, i, j) + q * 1024, 0, kDeviceScope);
                    }
            wait_vmcnt<0>();   // the partial has reached device scope before the count
            int before = 0;
            if (lane == 0) before = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = __builtin_amdgcn_readfirstlane(before) == splits - 1;
        }
        if (!last) return false;
        asm volatile("" ::: "memory");   // the partial loads stay after the count that allowed them
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                Acc total = Acc{0};
                for (int part = 0; part < splits; ++part) {
                    if (part == c_part) {
                        total += sum[i][j];
                    } else {
#pragma unroll
                        for (int q = 0; q < QUARTERS; ++q) {
                            const floatx4 v = __builtin_bit_cast(
                                floatx4, __builtin_amdgcn_raw_buffer_load_b128(rs, part_off(part, i, j) + q * 1024, 0,
                                                                              kDeviceScope));
                            total[4 * q] += v[0];
                            total[4 * q + 1] += v[1];
                            total[4 * q + 2] += v[2];
                            total[4 * q + 3] += v[3];
                        }
                    }
                }
                sum[i][j] = total;
            }
        if (lane == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return true;
    };

    // Prologue: steps 0 .. S-2 (early refill: 0 .. S-1) in flight, step 0
    // landed, its first k-step read.
    constexpr bool ER = Cfg::EARLY_REFILL && !WS;
    constexpr int PRO = ER ? S : S - 1;   // steps the prologue issues
    // KTAIL 2 (S == 2): fix_first: step 0 is a tile's last K-step.  fix_pending:
    // a fix is loaded (or, in the prologue, due) and waits for the barrier
    // before its stage is read.  With early refill the prologue fills step 1
    // too; its fix, for the tile at (fx1_m0, fx1_n0), is loaded once step 0's
    // has been applied, and applied at step 0's barrier.
    bool fix_first = false, fix_pending = false;
    int fx1_m0 = 0, fx1_n0 = 0;
    if (!WS || producer) {
#pragma unroll
        for (int s = 0; s < PRO; ++s) {
            if constexpr (KFIX) {
                if (s == 0) {
                    fix_first = fill_is_last_kstep();
                    if (fix_first) fix_issue(f_m0, f_n0);
                } else {
                    fix_pending = fill_is_last_kstep();
                    fx1_m0 = f_m0;
                    fx1_n0 = f_n0;
                }
            }
#pragma unroll
            for (int q = 0; q < NQ; ++q) dma(s, q);
            fill_advance();
        }
        wait_vmcnt<(PRO - 1) * NQ>();
    }
    lds_barrier();
    GEMM_RELU_MARK(1)
    if constexpr (KFIX) {
        if (fix_first) fix_apply(0);
        if (ER && fix_pending) fix_issue(fx1_m0, fx1_n0);
    }
    if constexpr (WS) {
        if (producer) {
            // The producer side of the ring: in step g, refill the slot step
            // g-1 used (free since the last barrier) with step g+S-1, wait for
            // step g+1 to land, and meet the compute waves at the barrier they
            // pass before reading step g+1.  Same barrier count as theirs.
            for (int g = 0; g < steps; ++g) {
                const int slot_fill = (g + S - 1) & (S - 1);
#pragma unroll
                for (int q = 0; q < NQ; ++q) dma(slot_fill, q);
                fill_advance();
                wait_vmcnt<(S - 2) * NQ>();
                lds_barrier();
            }
            wait_vmcnt<0>();   // no LDS DMA may outlive the workgroup
            return;
        }
    }
#pragma unroll
    for (int u = 0; u < NF; ++u) read_unit(0, 0, 0, u);
    constexpr int NQC = WS ? 0 : NQ;   // DMAs a compute wave issues per step

    // In the last k-step of a K-step, BAR_T MFMAs (on fragments already in
    // registers) are issued before the barrier, so the matrix pipe stays busy
    // while the waves meet; the next step's fragment reads follow the barrier.
    // Measured at 8192^3 with 8 MFMAs per k-step: 1 / 2 / 3 / 4 before the
    // barrier gave +0.8 / +1.4 / +0.7 / +0.3% (2: +0.7% on a second machine);
    // with 32 16x16 MFMAs per k-step, 4 (64 MFMA-cycles, as 2 32x32 MFMAs):
    // 2 / 4 / 8 / 12 / 16 gave 0.591 / 0.589 / 0.593 / 0.615 / 0.627 ms.
    // Smaller wave tiles keep the barrier first.
    constexpr int BAR_T = (!WS && NMF >= 8) ? (MF == 16 ? 4 : 2) : 0;
    static_assert(BAR_T < NMF && NKS >= 2, "the barrier is inside the last k-step");
    // Work items are numbered 0 .. NF-1 (fragment reads) and NF .. NF+NQC-1
    // (DMAs).  In the first k-step they are issued alternately, a DMA first,
    // so the DMAs start early without delaying the reads.  Measured against
    // all reads first: +1.6% at 8192^3 (256 tile; +0.3% over all DMAs
    // first), +3.3% at 2048^3 (128 tile), +1.3% at 1024^3 and +0.8% on the
    // 64 x 16384 x 8192 bf16 shape (64 tile).
    //  Early refill (ER) moves the DMAs into the last k-step, after the
    //  barrier, alternating with the reads of the next stage: the barrier has
    //  just freed the slot this step read (every wave's reads of it are done),
    //  so step g+S can go there a k-step sooner than in step g+1's first
    //  k-step.  With two 16x16 k-steps per stage (BK = 64) the DMAs of the
    //  first k-step land only a few MFMAs before the barrier that waits for
    //  them; early refill gives them a whole k-step more: 0.591 against
    //  0.665 ms at 8192^3 on zeros (full clock).  With four 32x32 k-steps per
    //  stage it costs time (0.610 against 0.552 ms), so it is a per-tile
    //  choice.  After the barrier, alternating against all reads first: 1415
    //  against 1396 TFLOP/s at the power cap (all DMAs first: 1367).
    constexpr bool ALTERNATE = !WS;
    auto first_kstep_item = [](int u0) {
        constexpr int PAIRS = NQC < NF ? NQC : NF;
        if (!ALTERNATE) return u0;
        if (u0 < 2 * PAIRS) return (u0 & 1) ? u0 / 2 : NF + u0 / 2;
        return NQC > NF ? NF + (u0 - PAIRS) : u0 - PAIRS;
    };
    for (int g = 0; g < steps; ++g) {
        const int slot = g & (S - 1);
        const int slot_next = (g + 1) & (S - 1);
        // The slot the DMAs of this step fill: step g-1's (free since the last
        // barrier) with step g+S-1, or with early refill this step's own (free
        // from this step's barrier on) with step g+S.
        const int slot_fill = ER ? slot : (g + S - 1) & (S - 1);
        // KTAIL 2: the stage filled in this step (step g+1) is a tile's last
        // K-step; its straddling pieces are loaded now and rewritten at the
        // step barrier.  With early refill the stage filled after this step's
        // barrier (step g+2) is the one; its pieces are loaded right after that
        // barrier and rewritten at the next step's (the fix loads are vector
        // loads, so the barrier's vmcnt wait covers them).
        if constexpr (KFIX && !ER) {
            fix_pending = fill_is_last_kstep();
            if (fix_pending) fix_issue(f_m0, f_n0);
        }
        auto step_barrier = [&]() {
            if constexpr (!WS) wait_vmcnt<(S - 2) * NQ>();   // step g+1 landed (for this wave)
            lds_barrier();                                   // ... and for every wave
            if constexpr (KFIX) {
                if (fix_pending) fix_apply(slot_next);
                if constexpr (ER) {
                    fix_pending = fill_is_last_kstep();
                    if (fix_pending) fix_issue(f_m0, f_n0);
                }
            }
        };
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int cur = ks & 1, nxt = cur ^ 1;
            const bool last = ks == NKS - 1;
            if (last && BAR_T == 0) step_barrier();
            // (Raising the wave's issue priority for the first k-steps, s_setprio,
            // once measured +1%; with the current schedule it costs 1% at
            // 8192^3 and up to 2% on the smaller tiles, so it is not used.)
            // Work spread over this k-step's MFMAs: the next k-step's fragment
            // reads (from the next stage after the barrier) and, in the first
            // k-step (early refill: the last, after the reads), the DMAs that
            // refill slot_fill (in the order first_kstep_item gives).
            const bool dma_ks = ER ? last : ks == 0;
            const int n_items = NF + (dma_ks ? NQC : 0);
#pragma unroll
            for (int t = 0; t < NMF; ++t) {
                if (last && BAR_T > 0 && t == BAR_T) step_barrier();
                // Snake order over the blocks: each MFMA changes one operand
                // fragment from the one before (measured: about +0.4%).
                const int bi = t / FM, bj = (bi & 1) ? FM - 1 - t % FM : t % FM;
                acc[bi][bj] = mfma<DT, MF>(fa[cur][bi], fb[cur][bj], acc[bi][bj]);
                // This MFMA's share of the work items; in the last k-step they
                // (reads of the next stage) start at the barrier.
                const int t0 = last ? t - BAR_T : t, span = last ? NMF - BAR_T : NMF;
                if (t0 < 0) {
                    __builtin_amdgcn_sched_barrier(0);
                    continue;
                }
#pragma unroll
                for (int u0 = t0 * n_items / span; u0 < (t0 + 1) * n_items / span; ++u0) {
                    const int u = dma_ks ? first_kstep_item(u0) : u0;
                    if (u < NF) {
                        if (last) read_unit(nxt, slot_next, 0, u);
                        else read_unit(nxt, slot, ks + 1, u);
                    } else {
                        dma(slot_fill, u - NF);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (!WS && dma_ks) fill_advance();
        }
        if (++c_kt == c_kt_end) {
            // Fused epilogue of the finished unit: ReLU, round to the dtype,
            // masked store (with SPLITK, by the last part of the tile, after
            // the partial sums are combined); then start the next unit from zero.
            GEMM_RELU_MARK(2)
            bool store = true;
            if constexpr (SPLITK) {
                if (splits > 1) store = combine_parts(acc);
            }
            if (store) {
                bool staged = false;
                if constexpr (Cfg::C_STAGE_WAVE > 0) {
                    if (c_vec_ok == 2) {
                        uint8_t* strip = smem + Cfg::LDS_BYTES + wave * Cfg::C_STAGE_WAVE;
                        if constexpr (MF == 32)
                            store_tile_staged<DT>(C, acc, strip, lane, c_m0 + wm * WTM, c_n0 + wn * WTN, M, N);
                        else
                            store_tile_staged16<DT>(C, acc, strip, lane, c_m0 + wm * WTM, c_n0 + wn * WTN, M, N);
                        staged = true;
                    }
                }
                if (!staged) {
#pragma unroll
                    for (int i = 0; i < FN; ++i)
#pragma unroll
                        for (int j = 0; j < FM; ++j) {
                            const int mb = c_m0 + wm * WTM + j * MF, nb = c_n0 + wn * WTN + i * MF;
                            if constexpr (MF == 32)
                                store_block<DT>(C, acc[i][j], lane, mb, nb, M, N, c_vec_ok != 0);
                            else
                                store_block16<DT>(C, acc[i][j], lane, mb, nb, M, N, c_vec_ok != 0);
                        }
                }
            }
            GEMM_RELU_MARK(3)
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) acc[i][j] = Acc{0};
            if (++c_unit < n_units) {
                unit_info(c_unit, c_tile, c_part, c_kt, c_kt_end);
                tile_origin(c_tile, c_m0, c_n0);
            }
        }
    }
    wait_vmcnt<0>();   // no LDS DMA may outlive the workgroup
    GEMM_RELU_TIMELINE_END
}

// Instances.
// Large shapes: BK = 64 in 2 stages.  Against BK = 32 in 4 stages (the same
// 128 KiB of LDS) it halves the barriers per k and makes every A row piece a
// whole 128-byte line (one L2 request instead of two): +2.7% at 8192^3,
// measured in one process.  8 waves of 128x64 on 16x16x32 MFMAs with early
// refill: on N(0, 0.1^2) fp16 8192^3, where the board's power cap sets the
// clock, 1396 TFLOP/s at 1792 MHz against 1293 TFLOP/s at 1632 MHz for 8
// waves of 64x128 on 32x32x16 MFMAs (the mfma_form program, alternating runs
// of 2.5 s); on another box 1400 against 1291, where 64x128 waves on 16x16x32
// gave 1384.  On zeros (full clock) the
// 32x32 form is the faster one, 0.552 against 0.582 ms.  128x64 waves read B
// (the ds_read_b64_tr_b16 side) for 64 columns instead of 128.
using DmaTile256 = DmaConfig<256, 256, 64, 2, 2, 4, 4, 16, 16, false, 0, true, true, 16, true>;
// K % 64 != 0 (KTAIL 1): 64x128 waves, whose K-tail masks fit in 254 VGPRs
// (the 128x64 layout needs 256 and 12 bytes of scratch per lane).  KTAIL 2
// (K % 8 != 0) fits in 254 with 128x64 waves and takes DmaTile256.
using DmaTile256Tail = DmaConfig<256, 256, 64, 2, 4, 2, 4, 16, 16, false, 0, true, true, 16, true>;
// With 4-byte DMA lanes for B (K, N) rows of an even length but not a multiple
// of 8, BK = 32 in 4 stages; A keeps 16-byte lanes where K % 8 == 0.
using DmaTile256B4 = DmaConfig<256, 256, 32, 4, 4, 2, 4, 16, 4>;
using DmaTile256AB4 = DmaConfig<256, 256, 32, 4, 4, 2, 4, 4, 4>;
using DmaTile128 = DmaConfig<128, 128, 64, 4, 2, 2, 4>;   // mid shapes: 4 waves of 64x64
using DmaTile64 = DmaConfig<64, 64, 64, 8, 2, 2, 4>;      // small and skinny shapes: 4 waves of 32x32, 8 stages
// At most 64 rows and many columns (split-K, and unsplit from 256 such tiles
// on): 4 waves of 64x64, 4 stages.  Each tile reads 512 bytes of every B row.
// This is HBM streaming, where less in flight per CU and no XCD remap measured
// faster: on 64 x 65536 x 2048 bf16, 44.6 us against 48.7 for 8 stages with
// the remap (5-9% on five such shapes); 64 x 16384 x 8192 in 4 parts, 54.6
// against 55.1 us.
using DmaTile64x256 = DmaConfig<64, 256, 32, 4, 1, 4, 4, 16, 16, false, 0, true, false>;
// B given as B^T, (N, K) row-major.  The 256 tile on 16x16x32 with early
// refill: 1451 TFLOP/s at 1747 MHz against 1327 at 1498 MHz on 32x32x16 (64x128
// waves both, in the measurement above); 128x64 waves, as for B (K, N), gave
// 1402 against 1388 for 64x128 on another box.
using DmaTile256T = DmaConfig<256, 256, 64, 2, 2, 4, 4, 16, 16, true, 0, true, true, 16, true>;
using DmaTile128T = DmaConfig<128, 128, 64, 4, 2, 2, 4, 16, 16, true>;
using DmaTile64T = DmaConfig<64, 64, 64, 8, 2, 2, 4, 16, 16, true>;
// B^T rows give a 64x256 tile only 64 bytes per row per K-step; 4 stages with
// the remap measured best of 8 / 4 with / 4 without (64 x 65536 x 2048: 66.9
// against 70.5 and 71.1 us; 64 x 16384 x 8192 in 2 parts: 76.6 against 81.1 and
// 80.6).
using DmaTile64x256T = DmaConfig<64, 256, 32, 4, 1, 4, 4, 16, 16, true>;
// Wave-specialised: 8 compute waves of 64x64 and 4 DMA-only producer waves
// (12 waves, 3 per SIMD: the 256x256 tile's accumulators leave no room for a
// producer wave beside its compute waves).
using DmaTile256x128W = DmaConfig<256, 128, 32, 4, 4, 2, 4, 16, 16, false, 4>;
using DmaTile256x128WT = DmaConfig<256, 128, 32, 4, 4, 2, 4, 16, 16, true, 4>;
// Few output tiles and deep K: 32x32 tiles (4 times as many as 64x64 ones)
// with one compute wave and 4 producer waves.  The producers keep the DMA
// stream going while the compute wave works through its K-steps: on 512 x 512
// x 16384 fp16, 42 us against 65 us for the 64x64x64 8-stage instance, in
// one process (a single wave with no producers: 76 us; 8 stages instead of
// 4: no faster, so bytes in flight are not the limit).
using DmaTile32W = DmaConfig<32, 32, 64, 4, 1, 1, 4, 16, 16, false, 4>;
// The B^T forms of the two producer-wave tiles that take decode-like shapes
// (at most 64 rows) rotate each tile's K order (K_ROTATE): on 64 x 16384 x 8192
// bf16, 48.4 against 57.9 us for the 64x64 tile; 64 x 65536 x 2048 53.5 against
// 60.6, 16 x 32768 x 8192 91.5 against 107.6; the 32x32 tile 2-9% faster.
using DmaTile32WT = DmaConfig<32, 32, 64, 4, 1, 1, 4, 16, 16, true, 4, true, true, 32, false, true>;
// The 64x64x64 tile with its 4 compute waves and 4 producer waves, 4 stages:
// on 1024^3 fp16, 6.6-7.1 us against 7.8-8.3 us for DmaTile64 (8 stages, the
// compute waves loading), in one process with bit-identical C.
using DmaTile64W = DmaConfig<64, 64, 64, 4, 2, 2, 4, 16, 16, false, 4>;
using DmaTile64WT = DmaConfig<64, 64, 64, 4, 2, 2, 4, 16, 16, true, 4, true, true, 32, false, true>;
// The same for the 128x128x64 tile: on 2048^3 fp16, 19.3-20.1 us against
// 21.2-21.7 us for DmaTile128, in one process with bit-identical C.
using DmaTile128W = DmaConfig<128, 128, 64, 4, 2, 2, 4, 16, 16, false, 4>;
using DmaTile128WT = DmaConfig<128, 128, 64, 4, 2, 2, 4, 16, 16, true, 4>;

// ---------------------------------------------------------------- direct kernel

// One wave per 32x32 block of C, operands gathered straight from global memory
// with a bounds check per element.  No LDS, no alignment requirement beyond
// 2 bytes.  It is the general path for shapes the tiled kernels cannot take
// and a second, structurally different GPU implementation for the tests.
// B_NK: B is given as B^T, an (N, K) row-major array.
template <int DT, bool B_NK = false>
__global__ __launch_bounds__(64) void gemm_relu_direct(const uint16_t* __restrict__ A,
                                                       const uint16_t* __restrict__ B,
                                                       uint16_t* __restrict__ C, int M, int N, int K,
                                                       int tiles_m, int c_vec_ok)
{
    const int lane = threadIdx.x;
    const int tm = blockIdx.x % tiles_m;
    const int tn = blockIdx.x / tiles_m;
    const int m = tm * 32 + (lane & 31);
    const int n = tn * 32 + (lane & 31);
    const int kg = (lane >> 5) * 8;
    floatx16 acc = floatx16{0};
    for (int k0 = 0; k0 < K; k0 += 16) {
        uint32_t fa[4], fb[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            uint32_t lo_a = 0, hi_a = 0, lo_b = 0, hi_b = 0;
            const int k = k0 + kg + 2 * p;
            if (B_NK) {
                if (n < N && k < K) lo_a = B[(size_t)n * K + k];
                if (n < N && k + 1 < K) hi_a = B[(size_t)n * K + k + 1];
            } else {
                if (n < N && k < K) lo_a = B[(size_t)k * N + n];
                if (n < N && k + 1 < K) hi_a = B[(size_t)(k + 1) * N + n];
            }
            if (m < M && k < K) lo_b = A[(size_t)m * K + k];
            if (m < M && k + 1 < K) hi_b = A[(size_t)m * K + k + 1];
            fa[p] = lo_a | (hi_a << 16);
            fb[p] = lo_b | (hi_b << 16);
        }
        acc = mfma_32x32x16<DT>(u32x4{fa[0], fa[1], fa[2], fa[3]}, u32x4{fb[0], fb[1], fb[2], fb[3]}, acc);
    }
    store_block<DT>(C, acc, lane, tm * 32, tn * 32, M, N, c_vec_ok != 0);
}

// Fill C (M x N) with +0.0: the result for K == 0 (an empty sum is 0, ReLU(0) = 0).
template <typename T>
__global__ void gemm_relu_zero_fill(T* __restrict__ C, size_t count)
{
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) C[i] = 0;
}

}  // namespace gemm_relu_hip
