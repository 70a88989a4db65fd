// C ABI of the gfx950 GEMM + ReLU library: argument checks, kernel choice and
// launch.  The operation and its contract are documented in gemm_relu.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/gemm_relu.h"
#include "kernel_table.hpp"

namespace gemm_relu_hip {
namespace {

constexpr int kVersion = 300;                    // 0.3.0
constexpr int64_t kMaxMN = int64_t(1) << 24;
constexpr int64_t kMaxK = int64_t(1) << 22;
constexpr int64_t kMaxBand = (int64_t(1) << 31) - 1;   // bytes one buffer descriptor may address
constexpr int kDirectTile = 32;

struct Plan {
    gemm_relu_config_t cfg;
    int tile;          // TileId, -1 direct kernel, -2 K == 0 fill, -4 an LDS-DMA kernel (dma_id)
    int dma_id;        // DmaId when tile == -4
    int dma_a4, dma_b4;    // 4-byte DMA lanes for A / B (256 LDS-DMA kernel, B stored (K, N) only)
    int kfix;              // 256 LDS-DMA kernel, 16-byte lanes, K even but not a multiple of 8 (KTAIL 2)
    int b_nk;          // B given as (N, K)
    int splits;        // K parts per tile (1: no split-K)
    int64_t counter_bytes;   // split-K workspace: per-tile counters, then the partial tiles
    int vec_pair;      // index into kVecPairs
    int tiles_m, tiles_n;
    int c_vec_ok;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Largest of 8, 4, 2, 1 elements that divides the row length and the pointer's
// alignment (in 2-byte elements).
int vec_width(const void* p, int64_t row_len)
{
    const uintptr_t addr = reinterpret_cast<uintptr_t>(p);
    for (int v = 8; v > 1; v /= 2)
        if (row_len % v == 0 && addr % (uintptr_t)(2 * v) == 0) return v;
    return 1;
}

bool overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes)
{
    if (a_bytes <= 0 || b_bytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)b_bytes && b0 < a0 + (uintptr_t)a_bytes;
}

// Every check that needs no device.  Fills `plan` on success.
// Split-K: the LDS-DMA instances that have split-K variants, and the number of
// work units that split-K aims for (one per CU of an MI355X).
bool has_splitk(int dma_id) { return dma_id == kDma128 || dma_id == kDma64 || dma_id == kDma64x256; }
constexpr int kSplitTargetUnits = 256;
constexpr int kMaxSplits = 64;
// The workspace starts with a counter region of fixed size, so that partial
// tiles of one call never land where another call (another shape) keeps its
// counters: counters, always reset to zero by the call that used them, stay
// zero from call to call whatever the shapes.
constexpr int64_t kCounterBytes = 65536;

// Shapes measured by tune.py on an MI355X: the fastest configuration of the
// plain entry points and of the split-K one.  The last row is a sentinel (M == 0
// never reaches the lookup).
struct TunedShape {
    int64_t m, n, k;
    int dtype, b_layout, config, splitk_config, splits;
};
constexpr TunedShape kTuned[] = {
#include "tuned_table.inc"
    {0, 0, 0, 0, 0, 0, 0, 0},
};

const TunedShape* find_tuned(int64_t M, int64_t N, int64_t K, int dtype, int b_layout)
{
    for (const TunedShape& t : kTuned)
        if (t.m == M && t.n == N && t.k == K && t.dtype == dtype && t.b_layout == b_layout) return &t;
    return nullptr;
}

// Widest load the row length allows (the width of aligned pointers).
int row_width(int64_t row_len)
{
    for (int v = 8; v > 1; v /= 2)
        if (row_len % v == 0) return v;
    return 1;
}

// splits_req: -1 for the entry points without a workspace (never split), 0 to
// choose, >= 1 to request that many K parts.
int make_plan(const void* A, const void* B, const void* C, int64_t M, int64_t N, int64_t K, int dtype,
              int b_layout, int config_id, int splits_req, Plan* plan)
{
    if (dtype != GEMM_RELU_F16 && dtype != GEMM_RELU_BF16) return GEMM_RELU_ERR_BAD_DTYPE;
    if (b_layout != GEMM_RELU_B_KN && b_layout != GEMM_RELU_B_NK) return GEMM_RELU_ERR_BAD_LAYOUT;
    if (M < 0 || N < 0 || K < 0) return GEMM_RELU_ERR_INVALID_ARG;
    if (config_id < GEMM_RELU_CONFIG_AUTO || config_id > GEMM_RELU_CONFIG_DMA_128x128_WS)
        return GEMM_RELU_ERR_BAD_CONFIG;
    if (splits_req < -1 || splits_req > kMaxSplits) return GEMM_RELU_ERR_INVALID_ARG;
    if (M > kMaxMN || N > kMaxMN || K > kMaxK) return GEMM_RELU_ERR_TOO_LARGE;

    std::memset(plan, 0, sizeof(*plan));
    plan->cfg.config_id = config_id;
    plan->cfg.b_layout = b_layout;
    plan->b_nk = b_layout == GEMM_RELU_B_NK ? 1 : 0;
    plan->splits = 1;
    plan->cfg.splits = 1;
    plan->tile = -3;
    if (M == 0 || N == 0) return GEMM_RELU_OK;        // nothing to compute or write

    // C is always written (K == 0 fills it with +0.0); A and B are read only when K > 0.
    const bool need_ab = K > 0;
    if (!C || (need_ab && (!A || !B))) return GEMM_RELU_ERR_INVALID_ARG;
    const uintptr_t odd = reinterpret_cast<uintptr_t>(C) | (need_ab ? (reinterpret_cast<uintptr_t>(A) |
                                                                      reinterpret_cast<uintptr_t>(B))
                                                                   : 0);
    if (odd & 1) return GEMM_RELU_ERR_MISALIGNED;
    const int64_t a_bytes = need_ab ? 2 * M * K : 0, b_bytes = need_ab ? 2 * K * N : 0;
    const int64_t c_bytes = 2 * M * N;
    if (overlaps(C, c_bytes, A, a_bytes) || overlaps(C, c_bytes, B, b_bytes)) return GEMM_RELU_ERR_ALIAS;

    const uintptr_t c_addr = reinterpret_cast<uintptr_t>(C);
    // 2: 16-byte pieces of C rows (the LDS-DMA kernels' staged stores), 1: 8-byte pieces, 0: elements.
    plan->c_vec_ok = (N % 8 == 0 && c_addr % 16 == 0) ? 2 : (N % 4 == 0 && c_addr % 8 == 0) ? 1 : 0;

    if (K == 0) {
        plan->tile = -2;
        plan->cfg.config_id = config_id;
        plan->cfg.threads = 256;
        plan->cfg.grid = std::min<int64_t>(ceil_div(M * N, 256), 65536);
        return GEMM_RELU_OK;
    }

    const int va = vec_width(A, K), vb = vec_width(B, plan->b_nk ? K : N);
    const bool full_vectors = va == 8 && vb == 8;
    // 4-byte DMA lanes work for rows of an even length with 4-byte aligned bases.
    const bool dword_vectors = va >= 2 && vb >= 2;
    int chosen = config_id;
    // A tuned shape, with pointers aligned as the tuner's were: its measured best.
    // An explicit number of parts keeps the tuned split-K tile only if that
    // tile has split-K kernels; otherwise the size rules below pick one that
    // does, so the request is never dropped.
    if (chosen == GEMM_RELU_CONFIG_AUTO && va == row_width(K) && vb == row_width(plan->b_nk ? K : N)) {
        if (const TunedShape* t = find_tuned(M, N, K, dtype, b_layout)) {
            if (splits_req < 0) {
                chosen = t->config;
            } else if (splits_req == 0) {
                chosen = t->splitk_config;
                splits_req = t->splits;
            } else if (t->splitk_config >= GEMM_RELU_CONFIG_DMA_256 &&
                       has_splitk(t->splitk_config - GEMM_RELU_CONFIG_DMA_256)) {
                chosen = t->splitk_config;
            }
        }
    }
    // With split-K on offer, a block of at most 64 rows takes the 64x256 tile:
    // its K parts restore the parallelism the few tiles lack.  Not for B stored
    // (N, K), where a 64x256 tile reads only 64 bytes of each B^T row per K-step
    // (the skinny shape in 2 parts: 76.6 us); the 64x64 tile takes it below.
    if (chosen == GEMM_RELU_CONFIG_AUTO && splits_req >= 0 && full_vectors && M <= 64 && !plan->b_nk)
        chosen = GEMM_RELU_CONFIG_DMA_64x256;
    // The plain entry point's small tiles take producer waves: 64x64 tiles
    // (measured faster at 1024^3), or, where 64x64 tiles would leave at least
    // half the CUs idle, 32x32 ones (4 times as many tiles; measured faster at
    // 256^3, 512^3 and 512 x 512 x 16384), since it has no workspace to split
    // K with.  The split-K entry point keeps the 64x64 tile without producers,
    // which has split-K instances, and splits K instead where it helps.
    // (With the parts left to the library, the split-K entry point splits only
    // below 192 tiles, so at or above that it takes the producer tiles too.)
    const int64_t t64 = ceil_div(M, 64) * ceil_div(N, 64);
    const bool few_tiles = t64 < 128;
    const int small_dma = splits_req > 0 || (splits_req == 0 && t64 < 192) ? GEMM_RELU_CONFIG_DMA_64
                          : few_tiles && splits_req < 0                   ? GEMM_RELU_CONFIG_DMA_32x32_WS
                                                                          : GEMM_RELU_CONFIG_DMA_64x64_WS;
    // 128x128 tiles run unsplit (192 or more of them) unless parts are asked
    // for: with producer waves (measured faster at 2048^3).
    const int mid_dma = splits_req > 0 ? GEMM_RELU_CONFIG_DMA_128 : GEMM_RELU_CONFIG_DMA_128x128_WS;
    if (plan->b_nk) {
        // B as (N, K): its rows are K-contiguous like A's.  The LDS-DMA kernels
        // need 16-byte lanes for both operands, or (the 256 one) 4-byte aligned
        // rows; otherwise (odd K, 2-byte alignment) the register-staged kernels,
        // which load B^T like A, take it.
        if (chosen == GEMM_RELU_CONFIG_AUTO) {
            const int64_t t256 = ceil_div(M, 256) * ceil_div(N, 256);
            const int64_t t128 = ceil_div(M, 128) * ceil_div(N, 128);
            // At most 64 rows: the small tiles whatever the tile count.  Their B^T
            // row pieces are as long as the larger tiles' and no tile rows are
            // wasted: 64 x 65536 x 2048 bf16 took 63.3 us against 78.7 on the 256
            // tile, 32 x 65536 x 4096 109 against 141, 16 x 32768 x 8192 111
            // against 127 on the 128x128 tile.
            if (!dword_vectors)
                chosen = t256 >= 192 ? GEMM_RELU_CONFIG_TILE_256 : GEMM_RELU_CONFIG_TILE_128;
            else if (M <= 64 && full_vectors)
                chosen = small_dma;
            else if (t256 >= 192 || !full_vectors)
                chosen = GEMM_RELU_CONFIG_DMA_256;
            else
                chosen = t128 >= 192 ? mid_dma : small_dma;
        }
        if ((chosen == GEMM_RELU_CONFIG_DMA_128 || chosen == GEMM_RELU_CONFIG_DMA_64 ||
             chosen == GEMM_RELU_CONFIG_DMA_64x256 || chosen == GEMM_RELU_CONFIG_DMA_256x128_WS ||
             chosen == GEMM_RELU_CONFIG_DMA_32x32_WS || chosen == GEMM_RELU_CONFIG_DMA_64x64_WS ||
             chosen == GEMM_RELU_CONFIG_DMA_128x128_WS) && !full_vectors && dword_vectors)
            chosen = GEMM_RELU_CONFIG_DMA_256;
    }
    if (chosen == GEMM_RELU_CONFIG_AUTO) {
        // The largest tile that still yields enough workgroups to cover the 256
        // CUs (192+ tiles); LDS-DMA kernels when 16-byte loads are possible (the
        // 256 tile also with 4-byte loads).  At most 64 rows over 256 or more
        // tiles of 64x256 stream B: the 64x256 tile reads 512 bytes of each B
        // row, wastes no rows, and measured 17-20% faster than the 256 tile on
        // 64 x 65536 x 2048 / 8192, 32 x 65536 x 4096 and 64 x 131072 x 4096 bf16
        // (below 256 such tiles, 128x128 ones were faster: 64 x 32768 x 4096).
        const int64_t t256 = ceil_div(M, 256) * ceil_div(N, 256);
        const int64_t t128 = ceil_div(M, 128) * ceil_div(N, 128);
        if (M <= 64 && full_vectors && ceil_div(N, 256) >= 256)
            chosen = GEMM_RELU_CONFIG_DMA_64x256;
        else if (t256 >= 192)
            chosen = dword_vectors ? GEMM_RELU_CONFIG_DMA_256 : GEMM_RELU_CONFIG_TILE_256;
        else if (full_vectors)
            chosen = t128 >= 192 ? mid_dma : small_dma;
        else
            chosen = GEMM_RELU_CONFIG_TILE_128;
    }
    if (chosen == GEMM_RELU_CONFIG_DMA_256 && !dword_vectors) chosen = GEMM_RELU_CONFIG_TILE_256;
    if ((chosen == GEMM_RELU_CONFIG_DMA_128 || chosen == GEMM_RELU_CONFIG_DMA_64 ||
         chosen == GEMM_RELU_CONFIG_DMA_64x256 || chosen == GEMM_RELU_CONFIG_DMA_32x32_WS ||
         chosen == GEMM_RELU_CONFIG_DMA_64x64_WS || chosen == GEMM_RELU_CONFIG_DMA_128x128_WS) && !full_vectors)
        chosen = GEMM_RELU_CONFIG_TILE_128;
    if (chosen == GEMM_RELU_CONFIG_DMA_256x128_WS && !full_vectors) chosen = GEMM_RELU_CONFIG_TILE_256;
    plan->cfg.config_id = chosen;

    if (chosen >= GEMM_RELU_CONFIG_DMA_256) {
        const int id = chosen - GEMM_RELU_CONFIG_DMA_256;
        // Lane widths.  The 256 kernel takes 16-byte lanes from any 4-byte
        // aligned rows (the other DMA tiles are only chosen with 16-byte aligned
        // rows of 8-element multiples).  Where K % 8 != 0, the K-contiguous row
        // pieces that straddle K (A, and B^T when B is stored (N, K)) are
        // rewritten in LDS by the KTAIL 2 instances, which need the 2-stage
        // ring.  B stored (K, N) with rows not of 8-element multiples takes
        // 4-byte lanes in a 4-stage ring of BK = 32, and then A does too where
        // K % 8 != 0.
        const bool b16 = plan->b_nk || vb == 8;
        const bool a16 = b16 || K % 8 == 0;
        const TileGeom& g = b16 ? kDmaGeom[id] : kDma256DwGeom;
        const int64_t b_band = plan->b_nk ? int64_t(g.bn) * K * 2 : int64_t(g.bk) * N * 2;
        if (int64_t(g.bm) * K * 2 > kMaxBand || b_band > kMaxBand) return GEMM_RELU_ERR_TOO_LARGE;
        const int64_t tm = ceil_div(M, g.bm), tn = ceil_div(N, g.bn);
        if (tm * tn > INT32_MAX) return GEMM_RELU_ERR_TOO_LARGE;
        plan->tile = -4;
        plan->dma_id = id;
        plan->tiles_m = (int)tm;
        plan->tiles_n = (int)tn;
        plan->cfg.block_m = g.bm;
        plan->cfg.block_n = g.bn;
        plan->cfg.block_k = g.bk;
        plan->cfg.stages = g.stages;
        plan->cfg.threads = g.threads;
        plan->dma_a4 = a16 ? 0 : 1;        // only the 256 kernel gets here with va or vb < 8
        plan->dma_b4 = b16 ? 0 : 1;
        plan->kfix = b16 && K % 8 != 0 ? 1 : 0;
        plan->cfg.vec_a = a16 ? 8 : 2;
        plan->cfg.vec_b = b16 ? 8 : 2;
        plan->cfg.grid = tm * tn;
        plan->cfg.lds_bytes = g.stages * (g.bm + g.bn) * g.bk * 2 + g.c_stage;
        if (splits_req >= 0 && has_splitk(id)) {
            const int64_t tiles = tm * tn, kt = ceil_div(K, g.bk);
            int64_t s = splits_req;
            if (s == 0) s = tiles >= 192 ? 1 : ceil_div(kSplitTargetUnits, tiles);
            s = std::min<int64_t>(s, std::min<int64_t>(kt, kMaxSplits));
            if (tiles * (g.threads / 64) * 4 > kCounterBytes) s = 1;   // one counter per tile and wave
            if (s > 1) {
                if (tiles * s > INT32_MAX) return GEMM_RELU_ERR_TOO_LARGE;
                plan->splits = (int)s;
                plan->counter_bytes = kCounterBytes;
                plan->cfg.splits = (int)s;
                plan->cfg.grid = tiles * s;
                plan->cfg.workspace_bytes = plan->counter_bytes + tiles * s * g.bm * g.bn * 4;
            }
        }
        return GEMM_RELU_OK;
    }

    if (chosen == GEMM_RELU_CONFIG_DIRECT) {
        const int64_t tm = ceil_div(M, kDirectTile), tn = ceil_div(N, kDirectTile);
        if (tm * tn > INT32_MAX) return GEMM_RELU_ERR_TOO_LARGE;
        plan->tile = -1;
        plan->tiles_m = (int)tm;
        plan->tiles_n = (int)tn;
        plan->cfg.block_m = kDirectTile;
        plan->cfg.block_n = kDirectTile;
        plan->cfg.threads = 64;
        plan->cfg.vec_a = 1;
        plan->cfg.vec_b = 1;
        plan->cfg.grid = tm * tn;
        return GEMM_RELU_OK;
    }

    const int tile = chosen == GEMM_RELU_CONFIG_TILE_256 ? kTile256 : kTile128;
    const TileGeom& g = kTileGeom[tile];
    // Each workgroup addresses A through a descriptor over bm rows and B through
    // one over bk rows (B stored (N, K): over bn rows of B^T); both must stay
    // below 2^31 bytes.
    const int64_t b_band = plan->b_nk ? int64_t(g.bn) * K * 2 : int64_t(g.bk) * N * 2;
    if (int64_t(g.bm) * K * 2 > kMaxBand || b_band > kMaxBand) return GEMM_RELU_ERR_TOO_LARGE;
    const int64_t tm = ceil_div(M, g.bm), tn = ceil_div(N, g.bn);
    if (tm * tn > INT32_MAX) return GEMM_RELU_ERR_TOO_LARGE;

    int pair = kNumVecPairs - 1;
    for (int i = 0; i < kNumVecPairs; ++i)
        if (kVecPairs[i][0] <= va && kVecPairs[i][1] <= vb) { pair = i; break; }

    plan->tile = tile;
    plan->vec_pair = pair;
    plan->tiles_m = (int)tm;
    plan->tiles_n = (int)tn;
    plan->cfg.block_m = g.bm;
    plan->cfg.block_n = g.bn;
    plan->cfg.block_k = g.bk;
    plan->cfg.stages = g.stages;
    plan->cfg.threads = g.threads;
    plan->cfg.vec_a = kVecPairs[pair][0];
    plan->cfg.vec_b = kVecPairs[pair][1];
    plan->cfg.grid = tm * tn;
    plan->cfg.lds_bytes = g.stages * (g.bm + g.bn) * g.bk * 2;
    return GEMM_RELU_OK;
}

// The split-K scratch of gemm_relu_splitk_noalloc: the fixed counter region,
// then room for the fp32 partial tiles.  One copy per device, held for the life
// of the process; every call on a device shares it.  In host code `scratch`
// names a host-side stand-in, never the device memory: kernels and copies get
// the address hipGetSymbolAddress returns for the current device.
constexpr int64_t kScratchBytes = GEMM_RELU_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes > kCounterBytes && kScratchBytes % 256 == 0, "scratch layout");
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[64];   // per device, under g_scratch_mutex

// The device address of this device's scratch array, looked up once per device
// with that device current.
int device_scratch(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GEMM_RELU_ERR_NO_DEVICE;
    if (dev >= 64) return GEMM_RELU_ERR_NO_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GEMM_RELU_ERR_LAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GEMM_RELU_OK;
}

// Per-device cache: 0 unknown, > 0 gfx950 with that many CUs, -1 something else.
std::atomic<int> g_device_cus[64];

// Checks that the current device is a gfx950 and returns its CU count in *cus.
int check_device(int* cus)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GEMM_RELU_ERR_NO_DEVICE;
    if (dev < 64) {
        const int known = g_device_cus[dev].load(std::memory_order_relaxed);
        if (known != 0) {
            *cus = known;
            return known > 0 ? GEMM_RELU_OK : GEMM_RELU_ERR_NO_DEVICE;
        }
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_RELU_ERR_NO_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 && prop.multiProcessorCount > 0;
    const int value = ok ? prop.multiProcessorCount : -1;
    if (dev < 64) g_device_cus[dev].store(value, std::memory_order_relaxed);
    *cus = value;
    return ok ? GEMM_RELU_OK : GEMM_RELU_ERR_NO_DEVICE;
}

int launch(const Plan& p, const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int dtype,
           int cus, void* workspace, hipStream_t stream)
{
    const DtypeKernels& ks = dtype == GEMM_RELU_F16 ? kernels_f16() : kernels_bf16();
    int m = (int)M, n = (int)N, k = (int)K;
    hipError_t err;
    if (p.tile == -2) {
        size_t count = (size_t)M * (size_t)N;
        void* args[] = {&C, &count};
        err = hipLaunchKernel(zero_fill_kernel(), dim3((unsigned)p.cfg.grid), dim3(256), args, 0, stream);
    } else if (p.tile == -1) {
        int tiles_m = p.tiles_m, c_vec_ok = p.c_vec_ok;
        void* args[] = {&A, &B, &C, &m, &n, &k, &tiles_m, &c_vec_ok};
        err = hipLaunchKernel(p.b_nk ? ks.direct_nt : ks.direct, dim3((unsigned)p.cfg.grid), dim3(64), args, 0,
                              stream);
    } else if (p.tile >= 0) {
        int tiles_m = p.tiles_m, tiles_n = p.tiles_n, c_vec_ok = p.c_vec_ok;
        void* args[] = {&A, &B, &C, &m, &n, &k, &tiles_m, &tiles_n, &c_vec_ok};
        const void* fn = p.b_nk ? ks.tiled_nt[p.tile][p.vec_pair] : ks.tiled[p.tile][p.vec_pair];
        err = hipLaunchKernel(fn, dim3((unsigned)p.cfg.grid), dim3((unsigned)p.cfg.threads), args, 0, stream);
    } else {
        int tiles_m = p.tiles_m, tiles_n = p.tiles_n, c_vec_ok = p.c_vec_ok, splits = p.splits;
        int* counters = p.splits > 1 ? static_cast<int*>(workspace) : nullptr;
        float* ws = p.splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + p.counter_bytes)
                                 : nullptr;
        void* args[] = {&A, &B, &C, &m, &n, &k, &tiles_m, &tiles_n, &c_vec_ok, &ws, &counters, &splits};
        const int ktail = K % p.cfg.block_k != 0 ? 1 : 0;
        const void* fn = p.splits > 1 ? ks.splitk[p.b_nk][p.dma_id][ktail]
                       : p.kfix ? (p.b_nk ? ks.dma_nt_kfix : ks.dma256_kfix)
                       : p.dma_b4 ? ks.dma256_b4[p.dma_a4][ktail]
                       : p.b_nk ? ks.dma_nt[p.dma_id][ktail] : ks.dma[p.dma_id][ktail];
        // The LDS-DMA kernels are persistent: one workgroup per CU (their LDS
        // ring fills a CU), each walking every grid-th work unit.
        const int64_t grid = std::min<int64_t>(p.cfg.grid, cus);
        err = hipLaunchKernel(fn, dim3((unsigned)grid), dim3((unsigned)p.cfg.threads), args, 0, stream);
    }
    return err == hipSuccess ? GEMM_RELU_OK : GEMM_RELU_ERR_LAUNCH;
}

int run(const Plan& p, const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int dtype,
        void* workspace, void* stream)
{
    if (p.tile == -3) return GEMM_RELU_OK;          // M == 0 or N == 0
    int cus = 0;
    const int rc = check_device(&cus);
    if (rc != GEMM_RELU_OK) return rc;
    return launch(p, A, B, C, M, N, K, dtype, cus, workspace, static_cast<hipStream_t>(stream));
}

}  // namespace
}  // namespace gemm_relu_hip

using namespace gemm_relu_hip;

extern "C" {

int gemm_relu_query_config_ex(const void* A, const void* B, const void* C, int64_t M, int64_t N, int64_t K,
                              int dtype, int b_layout, int config_id, gemm_relu_config_t* out)
{
    Plan p;
    const int rc = make_plan(A, B, C, M, N, K, dtype, b_layout, config_id, -1, &p);
    if (rc == GEMM_RELU_OK && out) *out = p.cfg;
    return rc;
}

int gemm_relu_query_config(const void* A, const void* B, const void* C, int64_t M, int64_t N, int64_t K,
                           int dtype, int config_id, gemm_relu_config_t* out)
{
    return gemm_relu_query_config_ex(A, B, C, M, N, K, dtype, GEMM_RELU_B_KN, config_id, out);
}

int gemm_relu_selected_config(int64_t M, int64_t N, int64_t K, int dtype, int* bm, int* bn, int* bk, int* stages)
{
    // gemm_relu's choice for dense 256-byte aligned, non-overlapping buffers
    // (what a device allocator returns).  The addresses are never dereferenced:
    // they only feed the alignment and overlap checks.
    const uintptr_t kBase = 256;
    auto round_up = [](int64_t bytes) { return (uintptr_t)((std::max<int64_t>(bytes, 0) + 255) / 256 * 256); };
    const uintptr_t a = kBase;
    const uintptr_t b = a + round_up(2 * M * K);
    const uintptr_t c = b + round_up(2 * K * N);
    Plan p;
    const int rc = make_plan(reinterpret_cast<const void*>(a), reinterpret_cast<const void*>(b),
                             reinterpret_cast<const void*>(c), M, N, K, dtype, GEMM_RELU_B_KN,
                             GEMM_RELU_CONFIG_AUTO, -1, &p);
    if (rc != GEMM_RELU_OK) return rc;
    if (bm) *bm = p.cfg.block_m;
    if (bn) *bn = p.cfg.block_n;
    if (bk) *bk = p.cfg.block_k;
    if (stages) *stages = p.cfg.stages;
    return GEMM_RELU_OK;
}

int gemm_relu_ex(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int dtype, int b_layout,
                 int config_id, void* stream)
{
    Plan p;
    const int rc = make_plan(A, B, C, M, N, K, dtype, b_layout, config_id, -1, &p);
    if (rc != GEMM_RELU_OK) return rc;
    return run(p, A, B, C, M, N, K, dtype, nullptr, stream);
}

int gemm_relu_with_config(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int dtype,
                          int config_id, void* stream)
{
    return gemm_relu_ex(A, B, C, M, N, K, dtype, GEMM_RELU_B_KN, config_id, stream);
}

int gemm_relu(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int dtype, void* stream)
{
    return gemm_relu_ex(A, B, C, M, N, K, dtype, GEMM_RELU_B_KN, GEMM_RELU_CONFIG_AUTO, stream);
}

int gemm_relu_query_splitk(const void* A, const void* B, const void* C, int64_t M, int64_t N, int64_t K, int dtype,
                           int b_layout, int config_id, int splits, gemm_relu_config_t* out)
{
    Plan p;
    const int rc = make_plan(A, B, C, M, N, K, dtype, b_layout, config_id, splits < 0 ? -2 : splits, &p);
    if (rc == GEMM_RELU_OK && out) *out = p.cfg;
    return rc;
}

int gemm_relu_splitk(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int dtype,
                     int b_layout, int config_id, int splits, void* workspace, int64_t workspace_bytes,
                     void* stream)
{
    Plan p;
    const int rc = make_plan(A, B, C, M, N, K, dtype, b_layout, config_id, splits < 0 ? -2 : splits, &p);
    if (rc != GEMM_RELU_OK) return rc;
    if (p.splits > 1) {
        if (!workspace || workspace_bytes < p.cfg.workspace_bytes ||
            reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
            return GEMM_RELU_ERR_WORKSPACE;
        const int64_t need = p.cfg.workspace_bytes;
        if (overlaps(workspace, need, C, 2 * M * N) || overlaps(workspace, need, A, 2 * M * K) ||
            overlaps(workspace, need, B, 2 * K * N))
            return GEMM_RELU_ERR_ALIAS;
    }
    return run(p, A, B, C, M, N, K, dtype, workspace, stream);
}

int gemm_relu_splitk_noalloc(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int dtype,
                             int b_layout, int config_id, int splits, void* stream)
{
    Plan p;
    const int rc = make_plan(A, B, C, M, N, K, dtype, b_layout, config_id, splits < 0 ? -2 : splits, &p);
    if (rc != GEMM_RELU_OK) return rc;
    if (p.splits <= 1) return run(p, A, B, C, M, N, K, dtype, nullptr, stream);
    if (p.cfg.workspace_bytes > kScratchBytes) return GEMM_RELU_ERR_SCRATCH;
    int cus = 0;
    int status = check_device(&cus);
    if (status != GEMM_RELU_OK) return status;
    void* ws = nullptr;
    status = device_scratch(&ws);
    if (status != GEMM_RELU_OK) return status;
    // The counters this call uses (one int per tile and wave) start at zero:
    // cleared by a fill kernel (not a memset node, so the call stays capturable),
    // ordered before the GEMM on the same stream.
    const hipStream_t s = static_cast<hipStream_t>(stream);
    size_t halves = (size_t)p.tiles_m * (size_t)p.tiles_n * (size_t)(p.cfg.threads / 64) * 2;
    void* fill_args[] = {&ws, &halves};
    const unsigned fill_grid = (unsigned)std::min<size_t>((halves + 255) / 256, 65536);
    if (hipLaunchKernel(zero_fill_kernel(), dim3(fill_grid), dim3(256), fill_args, 0, s) != hipSuccess)
        return GEMM_RELU_ERR_LAUNCH;
    return launch(p, A, B, C, M, N, K, dtype, cus, ws, s);
}

const char* gemm_relu_strerror(int code)
{
    switch (code) {
    case GEMM_RELU_OK: return "ok";
    case GEMM_RELU_ERR_INVALID_ARG: return "invalid argument (null pointer or negative dimension)";
    case GEMM_RELU_ERR_BAD_DTYPE: return "unsupported dtype (expected GEMM_RELU_F16 or GEMM_RELU_BF16)";
    case GEMM_RELU_ERR_ALIAS: return "C overlaps A or B";
    case GEMM_RELU_ERR_MISALIGNED: return "pointer not 2-byte aligned";
    case GEMM_RELU_ERR_NO_DEVICE: return "no current HIP device, or the device is not gfx950";
    case GEMM_RELU_ERR_LAUNCH: return "kernel launch failed";
    case GEMM_RELU_ERR_TOO_LARGE: return "dimensions exceed the supported range";
    case GEMM_RELU_ERR_BAD_CONFIG: return "unknown kernel configuration id";
    case GEMM_RELU_ERR_BAD_LAYOUT: return "unknown B layout (expected GEMM_RELU_B_KN or GEMM_RELU_B_NK)";
    case GEMM_RELU_ERR_WORKSPACE: return "split-K workspace missing, too small or not 256-byte aligned";
    case GEMM_RELU_ERR_SCRATCH:
        return "split-K partials of this call exceed the library's static scratch (gemm_relu_splitk_noalloc)";
    default: return "unknown error code";
    }
}

int gemm_relu_version(void) { return kVersion; }

}  // extern "C"
