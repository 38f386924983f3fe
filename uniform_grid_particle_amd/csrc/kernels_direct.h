// kernels_direct.h -- the direct (global-atomic) index build, used when the
// tile paths do not apply (more than 2^26 cell keys, or a bucketed tile
// would exceed 2^14 cells), plus the stand-alone scan.
//
// These follow the pages' chain closely: a clear, a count kernel with one
// device-scope atomicAdd per particle on conteos, a prefix scan, and a
// scatter with one returning atomic per particle on a cursor (pages
// "Contar partículas por celda", section "El kernel"; "Construir el índice
// de la rejilla con un prefix sum", sections "Del conteo al inicio" and
// "La dispersión"). The scan needs no look-back: the count kernel also sums,
// per workgroup in LDS, how many particles fall in each scan tile of
// 2^bin_shift cells and adds those partial sums with one global atomic per
// touched tile; every scan workgroup then adds the tile totals before its
// own tile. The cursor is initialised to inicios by the scan, so a slot is
// one returning atomic and conteos keeps the histogram.
#pragma once

#include "common.h"

namespace ugp {

constexpr int kCountItems = 8;       // particles per thread in count / scatter
constexpr int kScanItems = 16;       // consecutive cells per thread in the scan
constexpr uint32_t kScanSub = kBlock * kScanItems;  // 4096 cells per scan sub-tile
constexpr uint32_t kMaxBins = 512;   // scan tiles (LDS bins in count) upper bound
constexpr uint32_t kMinBinShift = 12;  // a scan tile is at least one sub-tile

// Zero `na` words of `a` (16-byte aligned) and `nb` words of `b`.
__global__ __launch_bounds__(kBlock) void clear_kernel(uint32_t* __restrict__ a, uint64_t na,
                                                        uint32_t* __restrict__ b, uint32_t nb) {
  const uint64_t nvec = na >> 2;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kBlock;
  uint4* av = reinterpret_cast<uint4*>(a);
  for (uint64_t v = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x; v < nvec; v += stride)
    av[v] = make_uint4(0u, 0u, 0u, 0u);
  if (blockIdx.x == 0) {
    for (uint64_t t = (nvec << 2) + threadIdx.x; t < na; t += kBlock) a[t] = 0u;
    for (uint32_t t = threadIdx.x; t < nb; t += kBlock) b[t] = 0u;
  }
}

// Count: one particle per (thread, item). Reads the 16-byte head of each
// 32-byte record (position + vida), writes celdaDe, adds to conteos with a
// non-returning device-scope atomic, and accumulates the per-scan-tile
// totals in LDS before one global atomic per touched tile.
__global__ __launch_bounds__(kBlock) void count_kernel(const float4* __restrict__ parts, uint32_t n,
                                                       GridParams g, uint32_t* __restrict__ celdaDe,
                                                       uint32_t* __restrict__ conteos,
                                                       uint32_t* __restrict__ tilesum,
                                                       uint32_t bin_shift, uint32_t nbins) {
  __shared__ uint32_t s_bins[kMaxBins];
  for (uint32_t b = threadIdx.x; b < nbins; b += kBlock) s_bins[b] = 0u;

  // Loads are unconditional (index clamped to n-1, n >= 1) so all of them
  // are in flight at once; only the uses are predicated.
  const uint32_t base = blockIdx.x * static_cast<uint32_t>(kBlock * kCountItems);
  float4 v[kCountItems];
#pragma unroll
  for (int j = 0; j < kCountItems; ++j) {
    const uint32_t i = base + j * kBlock + threadIdx.x;
    v[j] = parts[static_cast<size_t>(i < n ? i : n - 1u) * 2u];
  }
  __syncthreads();  // s_bins zeroed
#pragma unroll
  for (int j = 0; j < kCountItems; ++j) {
    const uint32_t i = base + j * kBlock + threadIdx.x;
    if (i < n) {
      const uint32_t c = cell_of(v[j].x, v[j].y, v[j].z, g);
      celdaDe[i] = c;
      atomicAdd(&conteos[c], 1u);
      atomicAdd(&s_bins[c >> bin_shift], 1u);
    }
  }
  __syncthreads();
  for (uint32_t b = threadIdx.x; b < nbins; b += kBlock) {
    const uint32_t cnt = s_bins[b];
    if (cnt) atomicAdd(&tilesum[b], cnt);
  }
}

// Per-tile sums for the standalone scan (no count kernel before it).
__global__ __launch_bounds__(kBlock) void tile_reduce_kernel(const uint32_t* __restrict__ in,
                                                             uint64_t count, uint32_t bin_shift,
                                                             uint32_t* __restrict__ tilesum) {
  __shared__ uint32_t s_wave[kBlock / 64];
  const uint64_t start = static_cast<uint64_t>(blockIdx.x) << bin_shift;
  uint64_t end = start + (1ull << bin_shift);
  if (end > count) end = count;
  uint32_t acc = 0;
  for (uint64_t i = start + threadIdx.x; i < end; i += kBlock) acc += in[i];
  uint32_t total;
  (void)block_exclusive_sum<kBlock>(acc, s_wave, &total);
  if (threadIdx.x == 0) tilesum[blockIdx.x] = total;
}

// Scan: workgroup t owns cells [t << bin_shift, (t+1) << bin_shift). Its
// offset is the sum of the tile totals before it; inside, sub-tiles of
// 4096 cells are scanned with 16 consecutive cells per thread. The last
// workgroup writes the grand total into the extra slot.
__global__ __launch_bounds__(kBlock) void scan_kernel(const uint32_t* __restrict__ in,
                                                      uint64_t count,
                                                      const uint32_t* __restrict__ tilesum,
                                                      uint32_t bin_shift,
                                                      uint32_t* __restrict__ out,
                                                      uint32_t* __restrict__ cursor) {
  __shared__ uint32_t s_wave[kBlock / 64];
  const uint32_t tile = blockIdx.x;
  uint32_t acc = 0;
  for (uint32_t b = threadIdx.x; b < tile; b += kBlock) acc += tilesum[b];
  uint32_t offset;
  (void)block_exclusive_sum<kBlock>(acc, s_wave, &offset);

  const uint64_t start = static_cast<uint64_t>(tile) << bin_shift;
  uint64_t end = start + (1ull << bin_shift);
  if (end > count) end = count;
  for (uint64_t sub = start; sub < end; sub += kScanSub) {
    const uint64_t my = sub + static_cast<uint64_t>(threadIdx.x) * kScanItems;
    const bool full = my + kScanItems <= end;
    uint32_t v[kScanItems];
    if (full) {
      const uint4* src = reinterpret_cast<const uint4*>(in + my);
#pragma unroll
      for (int q = 0; q < kScanItems / 4; ++q) {
        const uint4 w = src[q];
        v[4 * q + 0] = w.x;
        v[4 * q + 1] = w.y;
        v[4 * q + 2] = w.z;
        v[4 * q + 3] = w.w;
      }
    } else {
#pragma unroll
      for (int k = 0; k < kScanItems; ++k) v[k] = (my + k < end) ? in[my + k] : 0u;
    }
    uint32_t run = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
      const uint32_t c = v[k];
      v[k] = run;
      run += c;
    }
    uint32_t sub_total;
    const uint32_t excl = block_exclusive_sum<kBlock>(run, s_wave, &sub_total);
    const uint32_t add = offset + excl;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) v[k] += add;
    if (full) {
      uint4* dst = reinterpret_cast<uint4*>(out + my);
#pragma unroll
      for (int q = 0; q < kScanItems / 4; ++q)
        dst[q] = make_uint4(v[4 * q + 0], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
      if (cursor) {
        uint4* cur = reinterpret_cast<uint4*>(cursor + my);
#pragma unroll
        for (int q = 0; q < kScanItems / 4; ++q)
          cur[q] = make_uint4(v[4 * q + 0], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < kScanItems; ++k) {
        if (my + k < end) {
          out[my + k] = v[k];
          if (cursor) cursor[my + k] = v[k];
        }
      }
    }
    offset += sub_total;
  }
  if (tile == gridDim.x - 1 && threadIdx.x == 0) out[count] = offset;
}

// Scatter: slot = atomicAdd(cursor[c], 1) (cursor starts at inicios[c]);
// ordenado[slot] = i; with MOVE the record is copied to reordered[slot].
// Bounds checks keep a misused stage sequence from writing out of range.
template <bool MOVE>
__global__ __launch_bounds__(kBlock) void scatter_kernel(const uint32_t* __restrict__ celdaDe,
                                                         uint32_t n, uint32_t cells,
                                                         uint32_t* __restrict__ cursor,
                                                         uint32_t* __restrict__ ordenado,
                                                         const uint4* __restrict__ src,
                                                         uint4* __restrict__ dst) {
  const uint32_t base = blockIdx.x * static_cast<uint32_t>(kBlock * kCountItems);
  uint32_t c[kCountItems];
  uint4 ra[kCountItems], rb[kCountItems];
#pragma unroll
  for (int j = 0; j < kCountItems; ++j) {
    const uint32_t i = base + j * kBlock + threadIdx.x;
    const uint32_t ic = i < n ? i : n - 1u;  // unconditional loads, clamped index
    c[j] = celdaDe[ic];
    if (i >= n) c[j] = 0xFFFFFFFFu;
    if (MOVE) {
      ra[j] = src[static_cast<size_t>(ic) * 2u];
      rb[j] = src[static_cast<size_t>(ic) * 2u + 1u];
    }
  }
  uint32_t slot[kCountItems];
#pragma unroll
  for (int j = 0; j < kCountItems; ++j) {
    slot[j] = 0xFFFFFFFFu;
    if (c[j] < cells) slot[j] = atomicAdd(&cursor[c[j]], 1u);
  }
#pragma unroll
  for (int j = 0; j < kCountItems; ++j) {
    const uint32_t i = base + j * kBlock + threadIdx.x;
    if (slot[j] < n) {
      ordenado[slot[j]] = i;
      if (MOVE) {
        dst[static_cast<size_t>(slot[j]) * 2u] = ra[j];
        dst[static_cast<size_t>(slot[j]) * 2u + 1u] = rb[j];
      }
    }
  }
}

}  // namespace ugp
