// kernels_tiled.h -- the atomic-free index build (grids of up to 2^24 cells).
//
// On MI355X a device-scope global atomic is a memory-side transaction: a
// random u32 atomicAdd costs about as much HBM/fabric traffic as a 32-byte
// write and the atomic units bound the rate, so one atomic per particle per
// phase (the pages' count and scatter kernels) dominates the build. This
// path issues no global atomics. Cells are grouped into tiles of
// 2^tile_shift consecutive cell indices (4096..32768 cells, at most 512
// tiles), and the counting sort runs in two levels:
//
//   keys       per particle: cell key -> celdaDe; per workgroup: an LDS
//              histogram over tiles, stored as one row of a
//              [blocks x tiles] matrix (plain stores).
//   tile_scan  one workgroup per tile: exclusive scan of its column over
//              the blocks, in place, and the tile's total.
//   bucket     per workgroup: the tile starts (scan of the tile totals) plus
//              its own column offsets give an LDS cursor per tile; every
//              particle takes a slot with an LDS atomic and its (cell, index)
//              pair is written to that slot of the tile-ordered bucket array.
//   cells      one workgroup per tile: the tile's particles are counted into
//              an LDS histogram of its cells (conteos, written out), the
//              histogram is scanned in LDS (inicios, written out, offset by
//              the tile start), and every particle takes its final slot with
//              an LDS atomic: ordenado[slot] = index and, unless a separate
//              gather follows, reordered[slot] = particles[index].
//
// The result is the same counting sort: the histogram is exact, the starts
// are its exclusive scan, and every particle lands inside its cell's range;
// only the order inside a cell depends on LDS atomic arrival order, as the
// pages' atomic cursor does (page "Construir el índice de la rejilla con un
// prefix sum", section "El orden dentro de la celda").
#pragma once

#include "common.h"

namespace ugp {

constexpr uint32_t kMaxTiles = 512;        // tiles (LDS bins in keys / bucket)
constexpr uint32_t kTileShiftMin = 12;     // 4096 cells per tile at least
constexpr uint32_t kTileShiftMax = 15;     // 32768 cells (128 KiB LDS histogram) at most
constexpr int kCellsBlock = 1024;          // threads of the per-tile kernel
constexpr int kCellsBatch = 4;             // bucket entries per thread in flight

// keys: cell key per particle and the per-block tile histogram.
__global__ __launch_bounds__(kBlock) void tiled_keys_kernel(const float4* __restrict__ parts,
                                                            uint32_t n, GridParams g,
                                                            uint32_t* __restrict__ celdaDe,
                                                            uint32_t* __restrict__ hist,
                                                            uint32_t tile_shift, uint32_t ntiles,
                                                            uint32_t items) {
  __shared__ uint32_t s_hist[kMaxTiles];
  for (uint32_t t = threadIdx.x; t < ntiles; t += kBlock) s_hist[t] = 0u;
  __syncthreads();
  const uint64_t base = static_cast<uint64_t>(blockIdx.x) * kBlock * items;
  for (uint32_t b0 = 0; b0 < items; b0 += kBatch) {
    // unconditional loads (index clamped to n-1) so all are in flight at once
    float4 v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const uint64_t i = base + static_cast<uint64_t>(b0 + j) * kBlock + threadIdx.x;
      const uint64_t ic = i < n ? i : n - 1u;
      v[j] = parts[ic * 2u];
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const uint64_t i = base + static_cast<uint64_t>(b0 + j) * kBlock + threadIdx.x;
      if (i < n) {
        const uint32_t c = cell_of(v[j].x, v[j].y, v[j].z, g);
        celdaDe[i] = c;
        atomicAdd(&s_hist[c >> tile_shift], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t* row = hist + static_cast<size_t>(blockIdx.x) * ntiles;
  for (uint32_t t = threadIdx.x; t < ntiles; t += kBlock) row[t] = s_hist[t];
}

// tile_scan: block t scans column t of hist over the nblk rows, in place
// (exclusive), and writes the column total to tile_total[t].
__global__ __launch_bounds__(kBlock) void tiled_colscan_kernel(uint32_t* __restrict__ hist,
                                                               uint32_t nblk, uint32_t ntiles,
                                                               uint32_t* __restrict__ tile_total) {
  __shared__ uint32_t s_wave[kBlock / 64];
  const uint32_t t = blockIdx.x;
  uint32_t carry = 0;
  for (uint32_t w0 = 0; w0 < nblk; w0 += kBlock * 4) {
    uint32_t v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w = w0 + threadIdx.x * 4 + q;
      v[q] = (w < nblk) ? hist[static_cast<size_t>(w) * ntiles + t] : 0u;
    }
    const uint32_t sum = v[0] + v[1] + v[2] + v[3];
    uint32_t total;
    uint32_t run = carry + block_exclusive_sum<kBlock>(sum, s_wave, &total);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w = w0 + threadIdx.x * 4 + q;
      if (w < nblk) hist[static_cast<size_t>(w) * ntiles + t] = run;
      run += v[q];
    }
    carry += total;
  }
  if (threadIdx.x == 0) tile_total[t] = carry;
}

// bucket: place every particle's (cell, index) pair at its tile-ordered slot.
__global__ __launch_bounds__(kBlock) void tiled_bucket_kernel(const uint32_t* __restrict__ celdaDe,
                                                              uint32_t n,
                                                              const uint32_t* __restrict__ hist,
                                                              const uint32_t* __restrict__ tile_total,
                                                              uint32_t tile_shift, uint32_t ntiles,
                                                              uint32_t items,
                                                              uint2* __restrict__ bucket) {
  static_assert(kMaxTiles == 2 * kBlock, "two tiles per thread in the tile-start scan");
  __shared__ uint32_t s_off[kMaxTiles];
  __shared__ uint32_t s_wave[kBlock / 64];
  const uint32_t t0 = 2 * threadIdx.x;
  const uint32_t t1 = t0 + 1;
  const uint32_t a = t0 < ntiles ? tile_total[t0] : 0u;
  const uint32_t b = t1 < ntiles ? tile_total[t1] : 0u;
  uint32_t total;
  const uint32_t ex = block_exclusive_sum<kBlock>(a + b, s_wave, &total);
  const uint32_t* row = hist + static_cast<size_t>(blockIdx.x) * ntiles;
  if (t0 < ntiles) s_off[t0] = ex + row[t0];
  if (t1 < ntiles) s_off[t1] = ex + a + row[t1];
  __syncthreads();
  const uint64_t base = static_cast<uint64_t>(blockIdx.x) * kBlock * items;
  for (uint32_t b0 = 0; b0 < items; b0 += kBatch) {
    uint32_t c[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const uint64_t i = base + static_cast<uint64_t>(b0 + j) * kBlock + threadIdx.x;
      c[j] = celdaDe[i < n ? i : n - 1u];
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const uint64_t i = base + static_cast<uint64_t>(b0 + j) * kBlock + threadIdx.x;
      if (i < n) {
        const uint32_t tile = c[j] >> tile_shift;
        if (tile < ntiles) {
          const uint32_t r = atomicAdd(&s_off[tile], 1u);
          if (r < n) bucket[r] = make_uint2(c[j], static_cast<uint32_t>(i));
        }
      }
    }
  }
}

// cells: the per-tile counting sort. Block t owns cells
// [t << SHIFT, (t+1) << SHIFT) and bucket entries [bs, be).
template <bool MOVE, uint32_t SHIFT>
__global__ __launch_bounds__(kCellsBlock) void tiled_cells_kernel(
    const uint2* __restrict__ bucket, const uint32_t* __restrict__ tile_total, uint32_t ntiles,
    uint32_t cells, uint32_t n, uint32_t* __restrict__ conteos, uint32_t* __restrict__ inicios,
    uint32_t* __restrict__ ordenado, const uint4* __restrict__ src, uint4* __restrict__ dst) {
  constexpr uint32_t kTileCells = 1u << SHIFT;
  constexpr uint32_t kPer = kTileCells / kCellsBlock;  // consecutive cells per thread in the scan
  static_assert(kPer >= 1 && kTileCells % kCellsBlock == 0, "tile must cover the workgroup");
  __shared__ uint32_t s_cnt[kTileCells];
  __shared__ uint32_t s_wave[kCellsBlock / 64];
  const uint32_t t = blockIdx.x;
  const uint32_t cell0 = t << SHIFT;
  const uint32_t tc = (cells - cell0 < kTileCells) ? cells - cell0 : kTileCells;

  const uint32_t prev = (threadIdx.x < t && threadIdx.x < ntiles) ? tile_total[threadIdx.x] : 0u;
  const uint32_t bs = block_sum<kCellsBlock>(prev, s_wave);
  uint32_t be = bs + tile_total[t];
  if (be > n) be = n;  // only reachable if stages ran out of order

  for (uint32_t j = threadIdx.x; j < kTileCells; j += kCellsBlock) s_cnt[j] = 0u;
  __syncthreads();
  for (uint32_t k0 = bs; k0 < be; k0 += kCellsBlock * kCellsBatch) {
    uint32_t loc[kCellsBatch];
#pragma unroll
    for (int j = 0; j < kCellsBatch; ++j) {
      const uint32_t k = k0 + j * kCellsBlock + threadIdx.x;
      loc[j] = (k < be) ? bucket[k].x - cell0 : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int j = 0; j < kCellsBatch; ++j)
      if (loc[j] < tc) atomicAdd(&s_cnt[loc[j]], 1u);
  }
  __syncthreads();

  // histogram out, then its exclusive scan (offset by the tile start)
  const uint32_t j0 = threadIdx.x * kPer;
  uint32_t sum = 0;
#pragma unroll 4
  for (uint32_t q = 0; q < kPer; ++q) {
    const uint32_t j = j0 + q;
    if (j < tc) {
      const uint32_t v = s_cnt[j];
      conteos[cell0 + j] = v;
      sum += v;
    }
  }
  uint32_t total;
  uint32_t run = bs + block_exclusive_sum<kCellsBlock>(sum, s_wave, &total);
#pragma unroll 4
  for (uint32_t q = 0; q < kPer; ++q) {
    const uint32_t j = j0 + q;
    if (j < tc) {
      const uint32_t v = s_cnt[j];
      s_cnt[j] = run;
      inicios[cell0 + j] = run;
      run += v;
    }
  }
  if (t == ntiles - 1 && threadIdx.x == 0) inicios[cells] = be;
  __syncthreads();

  // final slots
  for (uint32_t k0 = bs; k0 < be; k0 += kCellsBlock * kCellsBatch) {
    uint2 e[kCellsBatch];
#pragma unroll
    for (int j = 0; j < kCellsBatch; ++j) {
      const uint32_t k = k0 + j * kCellsBlock + threadIdx.x;
      e[j] = bucket[k < be ? k : be - 1u];
      if (k >= be) e[j].x = 0xFFFFFFFFu;
    }
    uint32_t slot[kCellsBatch];
#pragma unroll
    for (int j = 0; j < kCellsBatch; ++j) {
      const uint32_t l = e[j].x - cell0;
      slot[j] = (e[j].x != 0xFFFFFFFFu && l < tc) ? atomicAdd(&s_cnt[l], 1u) : 0xFFFFFFFFu;
    }
    if (MOVE) {
      uint4 ra[kCellsBatch], rb[kCellsBatch];
#pragma unroll
      for (int j = 0; j < kCellsBatch; ++j) {
        const uint32_t p = e[j].y < n ? e[j].y : n - 1u;
        ra[j] = src[static_cast<size_t>(p) * 2u];
        rb[j] = src[static_cast<size_t>(p) * 2u + 1u];
      }
#pragma unroll
      for (int j = 0; j < kCellsBatch; ++j) {
        if (slot[j] < n && e[j].y < n) {
          ordenado[slot[j]] = e[j].y;
          dst[static_cast<size_t>(slot[j]) * 2u] = ra[j];
          dst[static_cast<size_t>(slot[j]) * 2u + 1u] = rb[j];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < kCellsBatch; ++j)
        if (slot[j] < n) ordenado[slot[j]] = e[j].y;
    }
  }
}

}  // namespace ugp
