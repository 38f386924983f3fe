// kernels_bucket.h -- the index build for more particles than the staged
// path takes (n > 2^21) or more cells (keys up to 2^26): four kernels, no
// global atomics, every record moved with coalesced-by-tile stores.
//
// A tile is 2^shift consecutive cell keys (16 to 16384 cells, up to 4096
// tiles, sized so a tile holds about 4096 particles on average).
//
//   keys       one workgroup per block of particles (at most 256 blocks):
//              cell key per particle (celdaDe) and an LDS histogram over
//              the tiles, stored as one row of a [blocks x tiles] matrix.
//   tile_scan  one workgroup per tile: exclusive scan of its column over
//              the blocks, in place, and the tile's total.
//   bucket     the same blocks again: tile starts (scan of the totals) plus
//              the block's column give an LDS cursor per tile; each
//              particle takes a slot with an LDS atomic and its record and
//              index are written there, so every tile's particles end up
//              contiguous. Block 0 also writes one row {count, start} per
//              tile.
//   tile_sort  the staged tile kernel (kernels_staged.h) with one "chunk"
//              per tile: the tile's particles are one contiguous run at its
//              start, so no chunk rows and no source map are needed.
//
// Against the pages' chain this reads the records twice (keys, bucket) and
// the bucketed copy once; every access is coalesced or a run per (block,
// tile), where the pages' scatter and gather touch a random record per
// particle.
#pragma once

#include "common.h"

namespace ugp {

constexpr uint32_t kBucketMaxTiles = 4096;  // LDS bins (16 KiB) in keys and bucket
constexpr uint32_t kBucketBlocks = 256;     // blocks at most: the matrix stays small
constexpr int kBucketThreads = 1024;        // threads per block
constexpr int kBucketBatch = 4;             // particles per thread in flight

// keys: particles [blockIdx.x * per_block, ...) of n. diag, fix_counts,
// queue_hdr (or nullptr): the two overflow-diagnostic words, the two stable
// fix-up list lengths and the shared-round counters, zeroed here for the
// tile kernel.
__global__ __launch_bounds__(kBucketThreads) void bucket_keys_kernel(
    const uint4* __restrict__ parts, uint32_t n, uint32_t per_block, GridParams g,
    uint32_t* __restrict__ celdaDe, uint32_t* __restrict__ hist, uint32_t tile_shift,
    uint32_t ntiles, uint32_t* __restrict__ diag, uint32_t* __restrict__ fix_counts,
    uint32_t* __restrict__ queue_hdr) {
  __shared__ uint32_t s_hist[kBucketMaxTiles];
  for (uint32_t t = threadIdx.x; t < ntiles; t += kBucketThreads) s_hist[t] = 0u;
  if (diag != nullptr && blockIdx.x == 0 && threadIdx.x < 2) diag[threadIdx.x] = 0u;
  if (fix_counts != nullptr && blockIdx.x == 0 && threadIdx.x < 2) fix_counts[threadIdx.x] = 0u;
  if (queue_hdr != nullptr && blockIdx.x == 0)  // shared rounds: claimed slots and ready flags
    for (uint32_t j = threadIdx.x; j < kQueueHeader; j += kBucketThreads) queue_hdr[j] = 0u;
  __syncthreads();
  const uint64_t base = static_cast<uint64_t>(blockIdx.x) * per_block;
  const uint64_t end = (base + per_block < n) ? base + per_block : n;
  for (uint64_t i0 = base; i0 < end; i0 += static_cast<uint64_t>(kBucketThreads) * kBucketBatch) {
    float x[kBucketBatch], y[kBucketBatch], z[kBucketBatch];
#pragma unroll
    for (int j = 0; j < kBucketBatch; ++j) {  // unconditional loads, clamped index
      const uint64_t i = i0 + static_cast<uint64_t>(j) * kBucketThreads + threadIdx.x;
      const uint4 a = load_stream(parts + (i < end ? i : end - 1u) * 2u);
      x[j] = __uint_as_float(a.x);
      y[j] = __uint_as_float(a.y);
      z[j] = __uint_as_float(a.z);
    }
#pragma unroll
    for (int j = 0; j < kBucketBatch; ++j) {
      const uint64_t i = i0 + static_cast<uint64_t>(j) * kBucketThreads + threadIdx.x;
      if (i < end) {
        const uint32_t c = cell_of(x[j], y[j], z[j], g);
        celdaDe[i] = c;
        atomicAdd(&s_hist[c >> tile_shift], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t* row = hist + static_cast<size_t>(blockIdx.x) * ntiles;
  for (uint32_t t = threadIdx.x; t < ntiles; t += kBucketThreads) row[t] = s_hist[t];
}

// bucket: the same blocks as keys; hist holds the column-scanned matrix and
// tile_total the tile totals. Writes tile_rec/tile_idx in tile order and
// (block 0) rows[t] = {tile_total[t], start of tile t}. Every lane of a wave
// reaches the lane exchange below (no early exit), as the shuffles need.
__global__ __launch_bounds__(kBucketThreads) void bucket_records_kernel(
    const uint4* __restrict__ parts, const uint32_t* __restrict__ celdaDe, uint32_t n,
    uint32_t per_block, const uint32_t* __restrict__ hist, const uint32_t* __restrict__ tile_total,
    uint32_t tile_shift, uint32_t ntiles, uint4* __restrict__ tile_rec,
    uint32_t* __restrict__ tile_idx, uint2* __restrict__ rows) {
  constexpr uint32_t kPer = kBucketMaxTiles / kBucketThreads;  // tiles per thread in the start scan
  __shared__ uint32_t s_off[kBucketMaxTiles];
  __shared__ uint32_t s_wave[kBucketThreads / 64];
  uint32_t tot[kPer];
  uint32_t sum = 0;
#pragma unroll
  for (uint32_t q = 0; q < kPer; ++q) {
    const uint32_t t = threadIdx.x * kPer + q;
    tot[q] = (t < ntiles) ? tile_total[t] : 0u;
    sum += tot[q];
  }
  uint32_t all;
  uint32_t start = block_exclusive_sum<kBucketThreads>(sum, s_wave, &all);
  const uint32_t* col = hist + static_cast<size_t>(blockIdx.x) * ntiles;
#pragma unroll
  for (uint32_t q = 0; q < kPer; ++q) {
    const uint32_t t = threadIdx.x * kPer + q;
    if (t < ntiles) {
      s_off[t] = start + col[t];
      if (blockIdx.x == 0) rows[t] = make_uint2(tot[q], start);
    }
    start += tot[q];
  }
  __syncthreads();
  const uint64_t base = static_cast<uint64_t>(blockIdx.x) * per_block;
  const uint64_t end = (base + per_block < n) ? base + per_block : n;
  for (uint64_t i0 = base; i0 < end; i0 += static_cast<uint64_t>(kBucketThreads) * kBucketBatch) {
    uint32_t w[8][kBucketBatch], c[kBucketBatch];
#pragma unroll
    for (int j = 0; j < kBucketBatch; ++j) {
      const uint64_t i = i0 + static_cast<uint64_t>(j) * kBucketThreads + threadIdx.x;
      const uint64_t ic = (i < end) ? i : end - 1u;
      const uint4 a = load_stream(parts + ic * 2u);
      const uint4 b = load_stream(parts + ic * 2u + 1u);
      c[j] = celdaDe[ic];
      w[0][j] = a.x; w[1][j] = a.y; w[2][j] = a.z; w[3][j] = a.w;
      w[4][j] = b.x; w[5][j] = b.y; w[6][j] = b.z; w[7][j] = b.w;
    }
    const uint32_t lane = threadIdx.x & 63u, half = lane & 1u;
#pragma unroll
    for (int j = 0; j < kBucketBatch; ++j) {
      const uint64_t i = i0 + static_cast<uint64_t>(j) * kBucketThreads + threadIdx.x;
      const uint32_t tile = c[j] >> tile_shift;
      uint32_t slot = 0xFFFFFFFFu;  // none
      if (i < end && tile < ntiles) {
        slot = atomicAdd(&s_off[tile], 1u);
        if (slot < n)
          tile_idx[slot] = static_cast<uint32_t>(i);
        else
          slot = 0xFFFFFFFFu;
      }
      // the records go out with lanes 2m and 2m + 1 storing the two halves
      // of one record (that of lane m, then of lane 32 + m): each store
      // instruction touches 32 records instead of 64 (measured on 16.8M
      // particles into 4096 tiles: 605 -> 572 us for this kernel)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int src = h * 32 + static_cast<int>(lane >> 1);
        const uint32_t to = static_cast<uint32_t>(__shfl(static_cast<int>(slot), src));
        uint32_t v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = static_cast<uint32_t>(__shfl(static_cast<int>(w[q][j]), src));
        const uint4 part = half ? make_uint4(v[4], v[5], v[6], v[7]) : make_uint4(v[0], v[1], v[2], v[3]);
        if (to != 0xFFFFFFFFu) tile_rec[static_cast<size_t>(to) * 2u + half] = part;
      }
    }
  }
}

// tile_scan: block t scans column t of hist over the nblk rows, in place
// (exclusive), and writes the column total to tile_total[t].
__global__ __launch_bounds__(kBlock) void bucket_colscan_kernel(uint32_t* __restrict__ hist,
                                                                uint32_t nblk, uint32_t ntiles,
                                                                uint32_t* __restrict__ tile_total) {
  __shared__ uint32_t s_wave[kBlock / 64];
  const uint32_t t = blockIdx.x;
  uint32_t carry = 0;
  for (uint32_t w0 = 0; w0 < nblk; w0 += kBlock) {
    const uint32_t w = w0 + threadIdx.x;
    const uint32_t v = (w < nblk) ? hist[static_cast<size_t>(w) * ntiles + t] : 0u;
    uint32_t total;
    const uint32_t ex = block_exclusive_sum<kBlock>(v, s_wave, &total);
    if (w < nblk) hist[static_cast<size_t>(w) * ntiles + t] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) tile_total[t] = carry;
}

}  // namespace ugp
