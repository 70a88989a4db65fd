/*
 * gemm_relu.h -- C ABI of the MI355X (gfx950) fused GEMM + ReLU library.
 *
 * The operation is the GEMM + ReLU example of "Writing High-Performance
 * Kernels in TileLang" (atlascloud.ai, section "Let's write a GEMM"; also its
 * Korean edition and the matrix-multiply example of the devpress.csdn.net
 * TileLang introduction):
 *
 *     C[i][j] = cast( max( sum_{k < K} A[i][k] * B[k][j], 0 ) )
 *
 * with A of shape (M, K), B of shape (K, N) and C of shape (M, N), all dense
 * row-major (leading dimensions K, N and N), all of one 16-bit dtype.  Products
 * are accumulated in fp32; max(x, 0) is taken on the fp32 accumulator and gives
 * +0.0 for every x <= 0; the cast rounds to nearest, ties to even.  The example
 * allocates C itself and passes it in; this ABI does the same.
 *
 * Memory: A, B and C are device pointers owned by the caller (e.g. torch
 * allocations).  The library allocates nothing and keeps no state between
 * calls except a per-device cache of the device's architecture (split-K takes
 * a caller-owned workspace; its no-allocation variant uses a static device
 * array that the library's code object holds on each device).
 *
 * Streams: work is enqueued on `stream` (a hipStream_t; NULL means the null
 * stream) and the call returns without waiting.  C is complete once the
 * stream has been synchronised.  Calls on different streams that write the
 * same C race.  Every entry point enqueues kernel launches only (no memset, no
 * copy, no allocation), so calls can be captured into a HIP graph and replayed;
 * the first call on a device queries its properties, so make it before capture.
 *
 * Errors: every argument is checked before anything is launched; on an error
 * the return value is negative, nothing is launched and C is not touched.
 *
 * Limits: M, N, K >= 0; M, N <= 2^24, K <= 2^22; each of A, B and C must be
 * smaller than 2^31 bytes in a single 256-row, 64-k-row band (see
 * GEMM_RELU_ERR_TOO_LARGE); pointers 2-byte aligned.  The fastest kernels also
 * want K % 8 == 0, N % 8 == 0 and 16-byte aligned A and B; other inputs take
 * narrower loads, with identical results.
 */
#ifndef GEMM_RELU_H
#define GEMM_RELU_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype of A, B and C (all three share it). */
enum {
    GEMM_RELU_F16 = 0,  /* IEEE binary16 */
    GEMM_RELU_BF16 = 1  /* bfloat16 */
};

/* Return codes. */
enum {
    GEMM_RELU_OK = 0,
    GEMM_RELU_ERR_INVALID_ARG = -1, /* null pointer with work to do, negative dimension */
    GEMM_RELU_ERR_BAD_DTYPE = -2,   /* dtype is neither GEMM_RELU_F16 nor GEMM_RELU_BF16 */
    GEMM_RELU_ERR_ALIAS = -3,       /* C overlaps A or B */
    GEMM_RELU_ERR_MISALIGNED = -4,  /* a pointer is not 2-byte aligned */
    GEMM_RELU_ERR_NO_DEVICE = -5,   /* no current HIP device, or it is not gfx950 */
    GEMM_RELU_ERR_LAUNCH = -6,      /* the HIP runtime refused the launch */
    GEMM_RELU_ERR_TOO_LARGE = -7,   /* a dimension or an addressed band exceeds the limits above */
    GEMM_RELU_ERR_BAD_CONFIG = -8,  /* an unknown kernel configuration id */
    GEMM_RELU_ERR_BAD_LAYOUT = -9,  /* b_layout is neither GEMM_RELU_B_KN nor GEMM_RELU_B_NK */
    GEMM_RELU_ERR_WORKSPACE = -10,  /* split-K workspace missing, too small or not 256-byte aligned */
    GEMM_RELU_ERR_SCRATCH = -11     /* gemm_relu_splitk_noalloc: the call needs more than the
                                       library's static scratch (GEMM_RELU_NOALLOC_SCRATCH_BYTES) */
};

/* How B is stored (gemm_relu_ex).  The operation is C = ReLU(A @ B) with B of
 * shape (K, N) either way.
 *   GEMM_RELU_B_KN: B itself, (K, N) row-major (leading dimension N).
 *   GEMM_RELU_B_NK: B^T, an (N, K) row-major array Bt with B[k][n] = Bt[n][k]
 *                   (leading dimension K): the "transpose_B" GEMM, whose B
 *                   buffer is declared (N, K) with a (block_N, block_K) shared
 *                   tile in "TileLang Guide: Composable Tiled AI Kernel
 *                   Programming" (aifetchly blog, sections "Tiles as
 *                   First-Class Language Primitives" and "Step 1: Defining the
 *                   Composable Kernel"); the tile-level gemm of "Writing
 *                   High-Performance Kernels in TileLang" (atlascloud.ai,
 *                   section "Let's write a GEMM", its list of primitives)
 *                   takes the same transpose flag. */
enum {
    GEMM_RELU_B_KN = 0,
    GEMM_RELU_B_NK = 1
};

/* Kernel configuration ids for gemm_relu_with_config (GEMM_RELU_CONFIG_AUTO
 * lets the library choose, as gemm_relu does).  AUTO first looks the exact
 * shape (M, N, K, dtype, B layout) up in a table of shapes measured on an
 * MI355X by tiled_dense_gemm_relu_amd/tune.py (compiled in from
 * csrc/tuned_table.inc; it applies when A and B are aligned for the widest
 * loads their row lengths allow, as in the tuner), else it uses size rules. */
enum {
    GEMM_RELU_CONFIG_AUTO = -1,
    GEMM_RELU_CONFIG_DIRECT = 0,      /* one wave per 32x32 block, operands from global memory */
    GEMM_RELU_CONFIG_TILE_256 = 1,    /* 256x256x64 block tile, 4 waves, 2 LDS stages */
    GEMM_RELU_CONFIG_TILE_128 = 2,    /* 128x128x64 block tile, 4 waves, 2 LDS stages */
    GEMM_RELU_CONFIG_DMA_256 = 3,     /* 256x256x64 block tile, 8 waves, 2 LDS stages filled by
                                         direct-to-LDS loads, 16x16x32 MFMAs; with 4-byte DMA
                                         lanes (rows that are not 16-byte multiples) 256x256x32 in
                                         4 stages on 32x32x16 MFMAs */
    GEMM_RELU_CONFIG_DMA_128 = 4,     /* 128x128x64 block tile, 4 waves, 4 direct-to-LDS stages */
    GEMM_RELU_CONFIG_DMA_64 = 5,      /* 64x64x64 block tile, 4 waves, 8 direct-to-LDS stages
                                         (small, skinny and bandwidth-bound shapes) */
    GEMM_RELU_CONFIG_DMA_64x256 = 6,  /* 64x256x32 block tile, 4 waves, 4 direct-to-LDS stages
                                         (few rows, many columns: split-K, and M <= 64 with at
                                         least 256 such tiles) */
    GEMM_RELU_CONFIG_DMA_256x128_WS = 7, /* 256x128x32 block tile, 4 direct-to-LDS stages, wave-
                                         specialised: 8 compute waves and 4 waves that only load */
    GEMM_RELU_CONFIG_DMA_32x32_WS = 8, /* 32x32x64 block tile, 4 direct-to-LDS stages, one compute
                                         wave and 4 waves that only load (few output tiles, deep
                                         K: 4 times as many tiles as 64x64 ones, no workspace) */
    GEMM_RELU_CONFIG_DMA_64x64_WS = 9, /* 64x64x64 block tile, 4 direct-to-LDS stages, 4 compute
                                         waves and 4 waves that only load */
    GEMM_RELU_CONFIG_DMA_128x128_WS = 10 /* 128x128x64 block tile, 4 direct-to-LDS stages, 4 compute
                                         waves and 4 waves that only load */
    /* DMA_128, DMA_64, DMA_64x256 and the *_WS configs need 16-byte loads of A and B
       (K % 8 == 0, N % 8 == 0, 16-byte aligned A and B); DMA_256 also takes 4-byte aligned rows (K and N
       even, 4-byte aligned A and B), with 16-byte loads, except that a B stored (K, N) whose
       rows are not 16-byte multiples on 16-byte boundaries takes 4-byte loads, and A then
       does too where K % 8 != 0.  For other inputs a DMA_* request falls back to TILE_256
       (DMA_256, DMA_256x128_WS) or TILE_128 (DMA_128, DMA_64, DMA_64x256, DMA_32x32_WS,
       DMA_64x64_WS, DMA_128x128_WS). */
};

/* What a configuration is, for reports and tests. */
typedef struct {
    int config_id;    /* GEMM_RELU_CONFIG_* actually used */
    int block_m;      /* rows of C per workgroup */
    int block_n;      /* columns of C per workgroup */
    int block_k;      /* k depth of one LDS stage (0 for the direct kernel) */
    int stages;       /* LDS stages (0 for the direct kernel) */
    int threads;      /* threads per workgroup */
    int vec_a;        /* elements per global load of A (1, 2, 4 or 8) */
    int vec_b;        /* elements per global load of B */
    int64_t grid;     /* output tiles; workgroups launched, except for the DMA_* kernels, which
                         run one persistent workgroup per CU (at most one per tile) */
    int lds_bytes;    /* LDS per workgroup: the ring of stages, plus C staging for the LDS-DMA kernels */
    int b_layout;     /* GEMM_RELU_B_KN or GEMM_RELU_B_NK */
    int splits;       /* K parts per output tile (1: no split-K) */
    int64_t workspace_bytes;   /* split-K workspace needed (0 when splits == 1) */
} gemm_relu_config_t;

/*
 * C = ReLU(A @ B).  A: (M, K), B: (K, N), C: (M, N), row-major, `dtype`.
 * M == 0 or N == 0: returns GEMM_RELU_OK and launches nothing.
 * K == 0: C is filled with +0.0 (the empty sum is 0 and ReLU(0) = +0.0).
 */
int gemm_relu(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int dtype,
              void* stream);

/* Same as gemm_relu with a forced kernel configuration (GEMM_RELU_CONFIG_*).
 * The result is the same for every configuration on integer-valued inputs;
 * on real-valued inputs the fp32 summation order may differ. */
int gemm_relu_with_config(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                          int dtype, int config_id, void* stream);

/* The configuration gemm_relu would use for these arguments (pure host logic:
 * no device is touched).  `out` may be NULL.  Returns GEMM_RELU_OK or the
 * error gemm_relu would return for these arguments' shape, dtype or alignment.
 * The GEMM page's kernel factory takes the block sizes (block_M, block_N,
 * block_K) and the pipeline's stage count as explicit parameters ("Writing
 * High-Performance Kernels in TileLang", atlascloud.ai, section "Let's write a
 * GEMM"); here the library picks them per shape, and this call reports the
 * pick with everything else that depends on the pointers (load widths, grid). */
int gemm_relu_query_config(const void* A, const void* B, const void* C, int64_t M, int64_t N,
                           int64_t K, int dtype, int config_id, gemm_relu_config_t* out);

/* The block tile and stage count gemm_relu picks for an (M, N, K) problem of
 * `dtype`, for dense row-major A, B and C on 256-byte aligned, separate
 * allocations (what a device allocator returns): the block_M, block_N, block_K
 * and num_stages that the GEMM page's kernel factory takes as parameters
 * ("Writing High-Performance Kernels in TileLang", atlascloud.ai, section
 * "Let's write a GEMM").  block_k and stages are 0 for the direct kernel; for
 * K == 0 (a fill of +0.0) all four are 0.  Any output pointer may be NULL.
 * Pure host logic: no device is touched.  Returns GEMM_RELU_OK, or the error
 * gemm_relu would return for this shape and dtype (then the outputs are not
 * written).  gemm_relu_query_config gives the full record for given pointers. */
int gemm_relu_selected_config(int64_t M, int64_t N, int64_t K, int dtype, int* bm, int* bn, int* bk,
                              int* stages);

/*
 * C = ReLU(A @ B) with B stored as `b_layout` says (GEMM_RELU_B_*) and a kernel
 * configuration (GEMM_RELU_CONFIG_*, or GEMM_RELU_CONFIG_AUTO).  With
 * GEMM_RELU_B_KN it is gemm_relu_with_config.  With GEMM_RELU_B_NK, B points
 * to the (N, K) array B^T, whose rows are K-contiguous like A's: every kernel
 * reads it.  The DMA_* kernels other than DMA_256 need K % 8 == 0 with 16-byte
 * aligned A and B (else DMA_256 serves them); DMA_256 needs K even with 4-byte
 * aligned A and B (else TILE_256 serves it); TILE_256, TILE_128 and DIRECT
 * take any K and alignment, with loads along K as wide as K and the pointers
 * allow.  Results, limits (B^T's 256-row band must stay below 2^31 bytes),
 * memory, stream and error behaviour are those of gemm_relu;
 * GEMM_RELU_ERR_BAD_LAYOUT for an unknown b_layout.
 */
int gemm_relu_ex(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int dtype,
                 int b_layout, int config_id, void* stream);

/* gemm_relu_query_config for gemm_relu_ex's arguments. */
int gemm_relu_query_config_ex(const void* A, const void* B, const void* C, int64_t M, int64_t N,
                              int64_t K, int dtype, int b_layout, int config_id,
                              gemm_relu_config_t* out);

/*
 * Split-K: C = ReLU(A @ B) with the K range of every output tile cut into
 * `splits` contiguous parts that run as separate work units, for shapes with
 * too few output tiles to occupy every CU (a few rows and many columns, or
 * small squares).  The split-K idea is the GEMM analogue of the split/combine
 * decode of "Writing High-Performance Kernels in TileLang" (atlascloud.ai,
 * its MLA decode section: a num_split parameter and a combine step); ReLU is
 * applied once, after the parts are summed, because it does not distribute
 * over a sum.
 *
 * Each part accumulates its K range in fp32; the last part of a tile to finish
 * (decided per wave sub-tile, without any waiting) adds the others' fp32
 * partial tiles in part order (part 0 first), applies ReLU, rounds and stores C.  The sum order is fixed, so results are the same
 * run to run; on integer-valued inputs they equal gemm_relu's bit for bit, on
 * real-valued inputs they differ from it only by fp32 summation order.
 *
 * splits: 0 lets the library choose (with GEMM_RELU_CONFIG_AUTO, a shape in
 * the tuned table takes the table's tile and parts; otherwise enough parts for
 * about 256 work units when the tiles alone are fewer than 192, else 1);
 * n >= 1 asks for n parts.  Either is capped at the tile's number of K-steps
 * and at 64.  Only the DMA_128, DMA_64 and DMA_64x256 kernels split; with other
 * configurations, or when the count resolves to 1, the call is gemm_relu_ex
 * (workspace unused, may be NULL).  With GEMM_RELU_CONFIG_AUTO and n >= 1 the
 * tile is always one that splits: the tuned table's, if it splits, else by the
 * size rules, which take DMA_64x256 for M <= 64 when its loads are possible
 * and B is stored (K, N).
 *
 * workspace: device memory of at least gemm_relu_config_t.workspace_bytes
 * (from gemm_relu_query_splitk with the same arguments), 256-byte aligned,
 * owned by the caller, not overlapping A, B or C.  Its first 64 KiB hold int
 * counters (one per output tile and wave; shapes that would need more do not
 * split), the fp32 partial tiles follow.  The counter region must be zero
 * before the first use; every call that runs to completion leaves it at zero
 * again, so the same workspace serves later calls of any shape without
 * clearing.  Calls that may overlap in time (different streams) need different
 * workspaces.
 * Errors as gemm_relu_ex, plus GEMM_RELU_ERR_WORKSPACE, and
 * GEMM_RELU_ERR_INVALID_ARG for splits < 0 or > 64.
 */
int gemm_relu_splitk(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, int dtype,
                     int b_layout, int config_id, int splits, void* workspace, int64_t workspace_bytes,
                     void* stream);

/* The configuration gemm_relu_splitk would use (pure host logic), including
 * `splits` and `workspace_bytes`.  `out` may be NULL. */
int gemm_relu_query_splitk(const void* A, const void* B, const void* C, int64_t M, int64_t N, int64_t K,
                           int dtype, int b_layout, int config_id, int splits, gemm_relu_config_t* out);

/* Size of the device array gemm_relu_splitk_noalloc uses as its workspace: the
 * 64 KiB counter region plus 32 MiB of fp32 partial tiles. */
#define GEMM_RELU_NOALLOC_SCRATCH_BYTES ((int64_t)65536 + ((int64_t)32 << 20))

/*
 * gemm_relu_splitk without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The split-K partials and counters live
 * in a static device array of GEMM_RELU_NOALLOC_SCRATCH_BYTES that the library
 * holds on every device it runs on until the process ends; the call allocates
 * nothing and calls no allocating routine.  The caller still passes A, B and C.
 *
 * Arguments, results and errors are those of gemm_relu_splitk with the
 * workspace removed; a call whose gemm_relu_query_splitk workspace_bytes
 * exceed GEMM_RELU_NOALLOC_SCRATCH_BYTES returns GEMM_RELU_ERR_SCRATCH before
 * anything is launched (ask for fewer parts).  When the split resolves to 1
 * part the call is gemm_relu_ex and the array is not touched.  Each split call
 * first clears the counters it uses (a small fill kernel on `stream`, ordered
 * before the GEMM), so the array's previous contents never matter.
 *
 * The array is shared by every call on a device: calls that may overlap in
 * time on one device (different streams, or different host threads without
 * ordering) race and give wrong results; order them on one stream.  The first
 * call on a device looks up the array's address; make it before graph capture.
 */
int gemm_relu_splitk_noalloc(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                             int dtype, int b_layout, int config_id, int splits, void* stream);

/* A static, human-readable description of a return code.  The pages' GEMM
 * surfaces its failures at two points, when the kernel is built (layout and
 * fragment-shape errors) and when it runs (out-of-bounds accesses from a wrong
 * grid or K loop, shared memory over budget at launch) (zwxr.cn hands-on
 * TileLang article, sections 5.1 and 5.2).  This library has no build step at
 * call time: every such condition is checked on the host before anything is
 * launched and returned as one of the codes above, which this call names. */
const char* gemm_relu_strerror(int code);

/* Library version, major * 10000 + minor * 100 + patch. */
int gemm_relu_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_RELU_H */
