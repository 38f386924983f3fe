// kernels_neighbor.h -- a neighbour query that consumes the index: for each
// particle, the number of other particles within a radius among the 27
// cells around its cell (page "Construir el índice de la rejilla con un
// prefix sum", section "La dispersión", for walking one cell's slice
// [inicios[c], inicios[c+1]); page "Reordenar por celda y la coalescencia
// de memoria", sections "Qué cuesta la indirección" and "El orden de las
// celdas también importa", for the 27-cell loop and why the data order
// matters).
//
// One thread per query particle, the loop the pages describe, with the
// queries taken in cell order (thread k answers the particle at place k of
// the index), so that the 64 lanes of a wave share the same few 27-cell
// neighbourhoods and mostly read the same candidate at each step. Two data
// orders:
//   INDIRECT  particles in their original order; thread k's query is
//             particle ordenado[k], a cell's slice lists particle indices
//             (ordenado) and every candidate position is a scattered read
//             -- the indirection the reorder page prices.
//   reordered particles already in cell order (the build's `reordered`);
//             thread k's query is record k and a slice is a contiguous run
//             of records.
// Either way a query meets itself once, in its own cell's slice at place k,
// with the same arithmetic as any other candidate; that term is taken off
// at the end.
// With the linear numbering the three cells x-1..x+1 of one row are
// consecutive keys, so each of the 9 rows is one contiguous range; with
// Morton keys each of the 27 cells is its own range.
//
// The squared distance is (dx*dx + dy*dy) + dz*dz in binary32, dx = xj - xi,
// without contraction (the library is built with -ffp-contract=off), so the
// comparison with r^2 is decided exactly as in a sequential reference.
#pragma once

#include "common.h"

namespace ugp {

constexpr int kNeighborBlock = 256;
constexpr uint32_t kNeighborUnroll = 8;  // candidates per step of the contiguous loop

// 1 when candidate q lies within the radius of pi, decided as described above
__device__ __forceinline__ uint32_t within(float4 q, float4 pi, float r2) {
  const float dx = q.x - pi.x;
  const float dy = q.y - pi.y;
  const float dz = q.z - pi.z;
  const float d2 = dx * dx + dy * dy + dz * dz;
  return (d2 <= r2) ? 1u : 0u;
}

// Candidates of slice [s, e), the query included when it lies in the slice
// (the caller takes its own term off once): INDIRECT, the records
// ordenado[s..e-1] (an entry >= n counts nothing); otherwise the contiguous
// records s..e-1.
template <bool INDIRECT>
__device__ __forceinline__ uint32_t count_range(const float4* __restrict__ parts,
                                                const uint32_t* __restrict__ ordenado, uint32_t n,
                                                float4 pi, float r2, uint32_t s, uint32_t e) {
  e = (e < n) ? e : n;  // a slice never runs past the particle count
  uint32_t cnt = 0;
  if (INDIRECT) {
    const uint32_t* o = ordenado + s;
    const uint32_t len = (e > s) ? e - s : 0u;
    uint32_t t = 0;
    for (; t + kNeighborUnroll <= len; t += kNeighborUnroll) {  // indices, then records, in flight together
      uint32_t j[kNeighborUnroll];
      float4 c[kNeighborUnroll];
#pragma unroll
      for (uint32_t u = 0; u < kNeighborUnroll; ++u) j[u] = o[t + u];
#pragma unroll
      for (uint32_t u = 0; u < kNeighborUnroll; ++u) c[u] = parts[2u * static_cast<size_t>(j[u] < n ? j[u] : 0u)];
#pragma unroll
      for (uint32_t u = 0; u < kNeighborUnroll; ++u) cnt += (j[u] < n) ? within(c[u], pi, r2) : 0u;
    }
    for (; t < len; ++t) {
      const uint32_t j = o[t];
      if (j < n) cnt += within(parts[2u * static_cast<size_t>(j)], pi, r2);
    }
    return cnt;
  }
  const float4* q = parts + 2u * static_cast<size_t>(s);
  const uint32_t len = (e > s) ? e - s : 0u;
  uint32_t t = 0;
  for (; t + kNeighborUnroll <= len; t += kNeighborUnroll) {  // these candidates' loads in flight together
    float4 c[kNeighborUnroll];
#pragma unroll
    for (uint32_t u = 0; u < kNeighborUnroll; ++u) c[u] = q[2u * (t + u)];
#pragma unroll
    for (uint32_t u = 0; u < kNeighborUnroll; ++u) cnt += within(c[u], pi, r2);
  }
  for (; t < len; ++t) cnt += within(q[2u * t], pi, r2);
  return cnt;
}

// Thread k answers the particle at place k of the index: INDIRECT, particle
// i = ordenado[k] of `parts` (original order), written to counts[i] (an
// entry >= n is skipped); otherwise record k of `parts` (cell order),
// written to counts[k]. parts: n 32-byte records as float4 pairs. dims:
// cells per axis; inicios: the build's starts (K+1 entries).
template <bool INDIRECT, bool MORTON>
__global__ __launch_bounds__(kNeighborBlock) void neighbor_count_kernel(
    const float4* __restrict__ parts, uint32_t n, GridParams g, uint32_t ny, uint32_t nz,
    const uint32_t* __restrict__ inicios, const uint32_t* __restrict__ ordenado, float r2,
    uint32_t* __restrict__ counts) {
  const uint32_t k = blockIdx.x * kNeighborBlock + threadIdx.x;
  if (k >= n) return;
  const uint32_t i = INDIRECT ? ordenado[k] : k;  // the query's particle
  if (i >= n) return;
  const float4 pi = parts[2u * static_cast<size_t>(i)];
  const uint32_t kx = axis_cell(pi.x, g.ox, g.h, g.tx);
  const uint32_t ky = axis_cell(pi.y, g.oy, g.h, g.ty);
  const uint32_t kz = axis_cell(pi.z, g.oz, g.h, g.tz);
  const uint32_t x0 = kx ? kx - 1u : 0u, x1 = (kx + 1u < g.nx) ? kx + 1u : kx;
  const uint32_t y0 = ky ? ky - 1u : 0u, y1 = (ky + 1u < ny) ? ky + 1u : ky;
  const uint32_t z0 = kz ? kz - 1u : 0u, z1 = (kz + 1u < nz) ? kz + 1u : kz;
  uint32_t cnt = 0;
  bool self_seen = false;  // the query's own place k was among the candidates
  for (uint32_t z = z0; z <= z1; ++z) {
    for (uint32_t y = y0; y <= y1; ++y) {
      if (MORTON) {
        const uint32_t yz = (spread_bits3(y) << 1) | (spread_bits3(z) << 2);
        for (uint32_t x = x0; x <= x1; ++x) {
          const uint32_t key = spread_bits3(x) | yz;
          const uint32_t s = inicios[key], e = inicios[key + 1u];
          cnt += count_range<INDIRECT>(parts, ordenado, n, pi, r2, s, e);
          self_seen = self_seen || (s <= k && k < e);
        }
      } else {
        const uint32_t row = y * g.nx + z * g.nxy;
        const uint32_t s = inicios[row + x0], e = inicios[row + x1 + 1u];
        cnt += count_range<INDIRECT>(parts, ordenado, n, pi, r2, s, e);
        self_seen = self_seen || (s <= k && k < e);
      }
    }
  }
  // the query met itself once, at place k (INDIRECT: ordenado[k] = i), with
  // the same arithmetic as any other candidate; take that term off
  if (self_seen) cnt -= within(pi, pi, r2);
  counts[i] = cnt;
}

}  // namespace ugp
