// The kernel instances of the gfx950 GEMM + ReLU library for one dtype, as a
// table of kernel addresses for the C ABI (kernel_table.hpp).  Each dtype's
// translation unit (kernels_f16.hip, kernels_bf16.hip) instantiates
// make_table<dtype>() once; a new kernel configuration is added here, in one
// place for both dtypes.
#pragma once

#include "gemm_relu_kernels.hpp"
#include "kernel_table.hpp"

namespace gemm_relu_hip {
namespace instances {
using Tile256 = TileConfig<256, 256, 2, 2, 8>;
using Tile128 = TileConfig<128, 128, 2, 2, 8>;

template <class Cfg, int id>
constexpr bool geom_matches = Cfg::BM == kTileGeom[id].bm && Cfg::BN == kTileGeom[id].bn &&
                              Cfg::BK == kTileGeom[id].bk && Cfg::STAGES == kTileGeom[id].stages &&
                              Cfg::THREADS == kTileGeom[id].threads && Cfg::GROUP_M == kTileGeom[id].group_m;
static_assert(geom_matches<Tile256, kTile256> && geom_matches<Tile128, kTile128>,
              "host tile table out of date");
template <class Cfg, int id>
constexpr bool dma_geom_matches = Cfg::BM == kDmaGeom[id].bm && Cfg::BN == kDmaGeom[id].bn &&
                                  Cfg::BK == kDmaGeom[id].bk && Cfg::STAGES == kDmaGeom[id].stages &&
                                  Cfg::THREADS == kDmaGeom[id].threads && Cfg::GROUP_M == kDmaGeom[id].group_m &&
                                  Cfg::C_STAGE_BYTES == kDmaGeom[id].c_stage;
template <class Cfg>
constexpr bool dw_geom_matches = Cfg::BM == kDma256DwGeom.bm && Cfg::BN == kDma256DwGeom.bn &&
                                 Cfg::BK == kDma256DwGeom.bk && Cfg::STAGES == kDma256DwGeom.stages &&
                                 Cfg::THREADS == kDma256DwGeom.threads && Cfg::GROUP_M == kDma256DwGeom.group_m &&
                                 Cfg::C_STAGE_BYTES == kDma256DwGeom.c_stage;
static_assert(dw_geom_matches<DmaTile256B4> && dw_geom_matches<DmaTile256AB4>,
              "host geometry of the 4-byte-lane 256 instances out of date");
static_assert(dma_geom_matches<DmaTile256, kDma256> && dma_geom_matches<DmaTile256Tail, kDma256> &&
                  dma_geom_matches<DmaTile128, kDma128> &&
                  dma_geom_matches<DmaTile64, kDma64> && dma_geom_matches<DmaTile256T, kDma256> &&
                  dma_geom_matches<DmaTile128T, kDma128> &&
                  dma_geom_matches<DmaTile64T, kDma64> && dma_geom_matches<DmaTile64x256, kDma64x256> &&
                  dma_geom_matches<DmaTile64x256T, kDma64x256> && dma_geom_matches<DmaTile256x128W, kDma256x128W> &&
                  dma_geom_matches<DmaTile256x128WT, kDma256x128W> && dma_geom_matches<DmaTile32W, kDma32W> &&
                  dma_geom_matches<DmaTile32WT, kDma32W> && dma_geom_matches<DmaTile64W, kDma64W> &&
                  dma_geom_matches<DmaTile64WT, kDma64W> && dma_geom_matches<DmaTile128W, kDma128W> &&
                  dma_geom_matches<DmaTile128WT, kDma128W>,
              "host DMA tile geometry out of date");

template <int DT, class Cfg, bool B_NK = false>
void fill_row(const void** row)
{
    row[0] = (const void*)&gemm_relu_tiled<Cfg, DT, 8, 8, B_NK>;
    row[1] = (const void*)&gemm_relu_tiled<Cfg, DT, 4, 8, B_NK>;
    row[2] = (const void*)&gemm_relu_tiled<Cfg, DT, 8, 4, B_NK>;
    row[3] = (const void*)&gemm_relu_tiled<Cfg, DT, 4, 4, B_NK>;
    row[4] = (const void*)&gemm_relu_tiled<Cfg, DT, 2, 2, B_NK>;
    row[5] = (const void*)&gemm_relu_tiled<Cfg, DT, 1, 1, B_NK>;
}

template <int DT, class KN, class NK>
void fill_splitk(DtypeKernels& t, int id)
{
    t.splitk[0][id][0] = (const void*)&gemm_relu_dma<KN, DT, false, true>;
    t.splitk[0][id][1] = (const void*)&gemm_relu_dma<KN, DT, true, true>;
    t.splitk[1][id][0] = (const void*)&gemm_relu_dma<NK, DT, false, true>;
    t.splitk[1][id][1] = (const void*)&gemm_relu_dma<NK, DT, true, true>;
}

template <int DT>
DtypeKernels make_table()
{
    DtypeKernels t{};
    fill_row<DT, Tile256>(t.tiled[kTile256]);
    fill_row<DT, Tile128>(t.tiled[kTile128]);
    fill_row<DT, Tile256, true>(t.tiled_nt[kTile256]);
    fill_row<DT, Tile128, true>(t.tiled_nt[kTile128]);
    t.direct = (const void*)&gemm_relu_direct<DT>;
    t.dma[kDma256][0] = (const void*)&gemm_relu_dma<DmaTile256, DT, false>;
    t.dma[kDma256][1] = (const void*)&gemm_relu_dma<DmaTile256Tail, DT, true>;
    t.dma[kDma128][0] = (const void*)&gemm_relu_dma<DmaTile128, DT, false>;
    t.dma[kDma128][1] = (const void*)&gemm_relu_dma<DmaTile128, DT, true>;
    t.dma[kDma64][0] = (const void*)&gemm_relu_dma<DmaTile64, DT, false>;
    t.dma[kDma64][1] = (const void*)&gemm_relu_dma<DmaTile64, DT, true>;
    t.dma256_b4[0][0] = (const void*)&gemm_relu_dma<DmaTile256B4, DT, 0>;
    t.dma256_b4[0][1] = (const void*)&gemm_relu_dma<DmaTile256B4, DT, 1>;
    t.dma256_b4[1][0] = (const void*)&gemm_relu_dma<DmaTile256AB4, DT, 0>;
    t.dma256_b4[1][1] = (const void*)&gemm_relu_dma<DmaTile256AB4, DT, 1>;
    t.dma256_kfix = (const void*)&gemm_relu_dma<DmaTile256, DT, 2>;
    t.direct_nt = (const void*)&gemm_relu_direct<DT, true>;
    t.dma_nt[kDma256][0] = (const void*)&gemm_relu_dma<DmaTile256T, DT, false>;
    t.dma_nt[kDma256][1] = (const void*)&gemm_relu_dma<DmaTile256T, DT, true>;
    t.dma_nt[kDma128][0] = (const void*)&gemm_relu_dma<DmaTile128T, DT, false>;
    t.dma_nt[kDma128][1] = (const void*)&gemm_relu_dma<DmaTile128T, DT, true>;
    t.dma_nt[kDma64][0] = (const void*)&gemm_relu_dma<DmaTile64T, DT, false>;
    t.dma_nt[kDma64][1] = (const void*)&gemm_relu_dma<DmaTile64T, DT, true>;
    t.dma_nt_kfix = (const void*)&gemm_relu_dma<DmaTile256T, DT, 2>;
    t.dma[kDma64x256][0] = (const void*)&gemm_relu_dma<DmaTile64x256, DT, false>;
    t.dma[kDma64x256][1] = (const void*)&gemm_relu_dma<DmaTile64x256, DT, true>;
    t.dma_nt[kDma64x256][0] = (const void*)&gemm_relu_dma<DmaTile64x256T, DT, false>;
    t.dma_nt[kDma64x256][1] = (const void*)&gemm_relu_dma<DmaTile64x256T, DT, true>;
    t.dma[kDma256x128W][0] = (const void*)&gemm_relu_dma<DmaTile256x128W, DT, false>;
    t.dma[kDma256x128W][1] = (const void*)&gemm_relu_dma<DmaTile256x128W, DT, true>;
    t.dma_nt[kDma256x128W][0] = (const void*)&gemm_relu_dma<DmaTile256x128WT, DT, false>;
    t.dma_nt[kDma256x128W][1] = (const void*)&gemm_relu_dma<DmaTile256x128WT, DT, true>;
    t.dma[kDma32W][0] = (const void*)&gemm_relu_dma<DmaTile32W, DT, 0>;
    t.dma[kDma32W][1] = (const void*)&gemm_relu_dma<DmaTile32W, DT, 1>;
    t.dma_nt[kDma32W][0] = (const void*)&gemm_relu_dma<DmaTile32WT, DT, 0>;
    t.dma_nt[kDma32W][1] = (const void*)&gemm_relu_dma<DmaTile32WT, DT, 1>;
    t.dma[kDma64W][0] = (const void*)&gemm_relu_dma<DmaTile64W, DT, 0>;
    t.dma[kDma64W][1] = (const void*)&gemm_relu_dma<DmaTile64W, DT, 1>;
    t.dma_nt[kDma64W][0] = (const void*)&gemm_relu_dma<DmaTile64WT, DT, 0>;
    t.dma_nt[kDma64W][1] = (const void*)&gemm_relu_dma<DmaTile64WT, DT, 1>;
    t.dma[kDma128W][0] = (const void*)&gemm_relu_dma<DmaTile128W, DT, 0>;
    t.dma[kDma128W][1] = (const void*)&gemm_relu_dma<DmaTile128W, DT, 1>;
    t.dma_nt[kDma128W][0] = (const void*)&gemm_relu_dma<DmaTile128WT, DT, 0>;
    t.dma_nt[kDma128W][1] = (const void*)&gemm_relu_dma<DmaTile128WT, DT, 1>;
    fill_splitk<DT, DmaTile128, DmaTile128T>(t, kDma128);
    fill_splitk<DT, DmaTile64, DmaTile64T>(t, kDma64);
    fill_splitk<DT, DmaTile64x256, DmaTile64x256T>(t, kDma64x256);
    return t;
}
}  // namespace instances


}  // namespace gemm_relu_hip
