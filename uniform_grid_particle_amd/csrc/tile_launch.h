// tile_launch.h -- host launchers of the staged tile kernel
// (kernels_staged.h), one per (records moved, overflow diagnostics, stable
// order, single tile) variant, each switching over the tile shifts 4..14.
// Every variant is instantiated in one of the tile_sort_*.hip translation
// units (compiled in parallel); ugp.hip sees only these declarations.
#pragma once

#include <hip/hip_runtime.h>

#include "kernels_staged.h"

namespace ugp {

#define UGP_TILE_LAUNCH_PARAMS                                                                     \
  uint32_t shift, dim3 grid, hipStream_t s, const uint2 *rows, uint32_t nchunks, uint32_t chunk,    \
      uint32_t ntiles, GridParams g, uint32_t cells, uint32_t n, const uint4 *chunk_rec,           \
      const uint32_t *chunk_idx, uint32_t *conteos, uint32_t *inicios, uint32_t *ordenado,         \
      uint4 *dst, uint32_t cap, uint32_t *diag, FixLists fl, uint32_t *keys_out, TileQueue q,              \
      uint32_t packed

template <bool MOVE, bool DIAG, bool STABLE, bool SINGLE>
void launch_staged_cells(UGP_TILE_LAUNCH_PARAMS);

#ifdef UGP_TILE_LAUNCH_DEFINE
template <bool MOVE, bool DIAG, bool STABLE, bool SINGLE, uint32_t SHIFT>
void launch_staged_cells_at(dim3 grid, hipStream_t s, const uint2* rows, uint32_t nchunks,
                            uint32_t chunk, uint32_t ntiles, GridParams g, uint32_t cells, uint32_t n,
                            const uint4* chunk_rec, const uint32_t* chunk_idx, uint32_t* conteos,
                            uint32_t* inicios, uint32_t* ordenado, uint4* dst, uint32_t cap,
                            uint32_t* diag, FixLists fl, uint32_t* keys_out, TileQueue q, uint32_t packed) {
  launch((staged_cells_kernel<MOVE, DIAG, STABLE, SINGLE, SHIFT, kCellsThreads, kCellsWin>), grid,
                     dim3(kCellsThreads), 0, s, rows, nchunks, chunk, ntiles, g, cells, n, chunk_rec,
                     chunk_idx, conteos, inicios, ordenado, dst, cap, diag, fl, keys_out, q, packed);
}

template <bool MOVE, bool DIAG, bool STABLE, bool SINGLE>
void launch_staged_cells(UGP_TILE_LAUNCH_PARAMS) {
#define UGP_STAGED_CASE(S)                                                                       \
  case S:                                                                                        \
    launch_staged_cells_at<MOVE, DIAG, STABLE, SINGLE, S>(grid, s, rows, nchunks, chunk, ntiles, \
                                                          g, cells, n, chunk_rec, chunk_idx,     \
                                                          conteos, inicios, ordenado, dst, cap,  \
                                                          diag, fl, keys_out, q, packed);        \
    break;
  switch (shift) {
    UGP_STAGED_CASE(4)
    UGP_STAGED_CASE(5)
    UGP_STAGED_CASE(6)
    UGP_STAGED_CASE(7)
    UGP_STAGED_CASE(8)
    UGP_STAGED_CASE(9)
    UGP_STAGED_CASE(10)
    UGP_STAGED_CASE(11)
    UGP_STAGED_CASE(12)
    UGP_STAGED_CASE(13)
    default:
      UGP_STAGED_CASE(14)
  }
#undef UGP_STAGED_CASE
}

// the four (stable order, single tile) variants of one (MOVE, DIAG) pair
#define UGP_TILE_INSTANTIATE(M, D)                                        \
  template void launch_staged_cells<M, D, false, false>(UGP_TILE_LAUNCH_PARAMS); \
  template void launch_staged_cells<M, D, false, true>(UGP_TILE_LAUNCH_PARAMS);  \
  template void launch_staged_cells<M, D, true, false>(UGP_TILE_LAUNCH_PARAMS);  \
  template void launch_staged_cells<M, D, true, true>(UGP_TILE_LAUNCH_PARAMS);
#endif

}  // namespace ugp
