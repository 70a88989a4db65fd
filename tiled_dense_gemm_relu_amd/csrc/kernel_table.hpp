// Host-side table of the compiled kernel instances, filled by one translation
// unit per dtype.  The C ABI (gemm_relu_api.hip) looks kernels up here and
// launches them with hipLaunchKernel.
#pragma once

namespace gemm_relu_hip {

// Tile configurations, by GEMM_RELU_CONFIG_* id.
enum TileId { kTile256 = 0, kTile128 = 1, kNumTiles = 2 };

// Geometry of each tile configuration (must match the TileConfig instances).
struct TileGeom {
    int bm, bn, bk, stages, threads, group_m;
    int c_stage = 0;   // LDS bytes past the ring for staging C (LDS-DMA kernels)
};
constexpr TileGeom kTileGeom[kNumTiles] = {
    {256, 256, 64, 2, 256, 8},
    {128, 128, 64, 2, 256, 8},
};

// (vec_a, vec_b) pairs with a compiled instance, in order of preference.
constexpr int kNumVecPairs = 6;
constexpr int kVecPairs[kNumVecPairs][2] = {{8, 8}, {4, 8}, {8, 4}, {4, 4}, {2, 2}, {1, 1}};

// LDS-DMA kernel instances, by GEMM_RELU_CONFIG_DMA_* order.
enum DmaId {
    kDma256 = 0, kDma128 = 1, kDma64 = 2, kDma64x256 = 3, kDma256x128W = 4, kDma32W = 5, kDma64W = 6, kDma128W = 7,
    kNumDma = 8
};

struct DtypeKernels {
    // Register-staged kernels by TileId and load-width pair; tiled_nt reads B
    // given as B^T, an (N, K) row-major array (its load width counts along K).
    const void* tiled[kNumTiles][kNumVecPairs];
    const void* tiled_nt[kNumTiles][kNumVecPairs];
    const void* direct;
    const void* dma[kNumDma][2];   // LDS-DMA kernels by DmaId, [K % BK != 0]; need 8-element loads of A and B
    // The 256 LDS-DMA kernel with 4-byte DMA lanes for B (B rows of an even
    // length): [A 4-byte lanes][K % BK != 0].  A takes 16-byte lanes from any
    // 4-byte aligned row where K % 8 == 0, else 4-byte lanes.
    const void* dma256_b4[2][2];
    // The 256 LDS-DMA kernel with 16-byte lanes from 4-byte aligned rows and K
    // even but not a multiple of 8 (KTAIL 2: the piece straddling K is
    // rewritten in LDS); for B stored (K, N) B needs 8-element loads.
    const void* dma256_kfix;
    // B given as B^T, an (N, K) row-major array: the direct kernel, the
    // LDS-DMA kernels with 16-byte lanes by DmaId and [K % BK != 0], and the
    // 256 one with KTAIL 2.
    const void* direct_nt;
    const void* dma_nt[kNumDma][2];
    const void* dma_nt_kfix;
    // Split-K instances (8-element loads): [B layout][DmaId][K % BK != 0];
    // null for the 256 tiles, which have none.
    const void* splitk[2][kNumDma][2];
};

// Geometry of each LDS-DMA instance (must match DmaTile256 / DmaTile128 / DmaTile64 / DmaTile64x256 /
// DmaTile256x128W / DmaTile32W / DmaTile64W / DmaTile128W; threads include the producer waves).
constexpr TileGeom kDmaGeom[kNumDma] = {
    {256, 256, 64, 2, 512, 4, 32768},
    {128, 128, 64, 4, 256, 4, 16384},
    {64, 64, 64, 8, 256, 4, 0},
    {64, 256, 32, 4, 256, 4, 16384},
    {256, 128, 32, 4, 768, 4, 32768},
    {32, 32, 64, 4, 320, 4, 0},
    {64, 64, 64, 4, 512, 4, 0},
    {128, 128, 64, 4, 512, 4, 16384},
};
// The 256 instances with 4-byte DMA lanes keep BK = 32 in 4 stages: with four
// DMA instructions for every 16-byte one, the deeper ring measured about 4%
// faster (on 4000x11000x4100 with 4-byte A lanes).
constexpr TileGeom kDma256DwGeom = {256, 256, 32, 4, 512, 4, 32768};

const DtypeKernels& kernels_f16();
const DtypeKernels& kernels_bf16();
const void* zero_fill_kernel();

}  // namespace gemm_relu_hip
