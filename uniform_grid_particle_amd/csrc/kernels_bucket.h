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
//   tile_scan  one workgroup per 64 tiles: exclusive scan of each column
//              over the blocks, in place, and the tile totals.
//   bucket     the same blocks again: tile starts (scan of the totals) plus
//              the block's column give an LDS cursor per tile; each
//              particle takes a slot with an LDS atomic and its record is
//              written there, so every tile's particles end up contiguous;
//              the indices follow at the end, run by run, from an inverse
//              map in LDS. Block 0 also writes one row {count, start} per
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
constexpr uint32_t kBucketBlocks = 256;     // blocks sought: the matrix stays small
constexpr uint32_t kBucketMaxPerBlock = 1u << 16;  // particles per block at most (16-bit offsets in LDS)
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
// (block 0) rows[t] = {tile_total[t], start of tile t}.
//
// Records go out as they are placed (32 bytes each, whole 32-byte sectors).
// Indices would go out 4 bytes at a time into the ~16-word run of each
// (block, tile), the run's line filled over the whole pass and written back
// piecemeal; so the block keeps an inverse map in LDS instead (local
// position in tile order -> particle offset in the block, 16 bits) and
// writes every run of indices at the end, consecutive lanes to consecutive
// words. Local positions: the block's own counts (the difference of its row
// and the next in the scanned matrix) scanned over the tiles; tile t's
// local range [lbase_t, lbase_t + count) maps onto its slots
// [start_t + col_t, ...) by the offset s_d[t].
//
// Every lane of a wave reaches the lane exchange below (no early exit), as
// the shuffles need. per_block <= kBucketMaxPerBlock.
__global__ __launch_bounds__(kBucketThreads) void bucket_records_kernel(
    const uint4* __restrict__ parts, const uint32_t* __restrict__ celdaDe, uint32_t n,
    uint32_t per_block, const uint32_t* __restrict__ hist, const uint32_t* __restrict__ tile_total,
    uint32_t tile_shift, uint32_t ntiles, uint4* __restrict__ tile_rec,
    uint32_t* __restrict__ tile_idx, uint2* __restrict__ rows) {
  constexpr uint32_t kPer = kBucketMaxTiles / kBucketThreads;  // tiles per thread in the scans
  // 160 KiB: per tile a local cursor and a slot offset, then the inverse map
  // (whose first words also serve the scans before the map is written)
  __shared__ uint32_t s_lds[2 * kBucketMaxTiles + kBucketMaxPerBlock / 2];
  uint32_t* s_loc = s_lds;
  uint32_t* s_d = s_lds + kBucketMaxTiles;
  uint16_t* s_inv = reinterpret_cast<uint16_t*>(s_lds + 2 * kBucketMaxTiles);
  uint32_t* s_wave = s_lds + 2 * kBucketMaxTiles;

  const uint32_t* col = hist + static_cast<size_t>(blockIdx.x) * ntiles;
  const uint32_t* next = (blockIdx.x + 1u == gridDim.x) ? tile_total : col + ntiles;
  uint32_t tot[kPer], cnt[kPer], c0[kPer];
  uint32_t sum = 0, lsum = 0;
#pragma unroll
  for (uint32_t q = 0; q < kPer; ++q) {
    const uint32_t t = threadIdx.x * kPer + q;
    tot[q] = (t < ntiles) ? tile_total[t] : 0u;
    c0[q] = (t < ntiles) ? col[t] : 0u;
    cnt[q] = (t < ntiles) ? next[t] - c0[q] : 0u;
    sum += tot[q];
    lsum += cnt[q];
  }
  uint32_t all;
  uint32_t start = block_exclusive_sum<kBucketThreads>(sum, s_wave, &all);
  uint32_t lbase = block_exclusive_sum<kBucketThreads>(lsum, s_wave, &all);
#pragma unroll
  for (uint32_t q = 0; q < kPer; ++q) {
    const uint32_t t = threadIdx.x * kPer + q;
    if (t < ntiles) {
      s_loc[t] = lbase;
      s_d[t] = start + c0[q] - lbase;  // modulo 2^32: slot = local + s_d
      if (blockIdx.x == 0) rows[t] = make_uint2(tot[q], start);
    }
    start += tot[q];
    lbase += cnt[q];
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
        const uint32_t local = atomicAdd(&s_loc[tile], 1u);
        if (local < kBucketMaxPerBlock) s_inv[local] = static_cast<uint16_t>(i - base);
        slot = local + s_d[tile];
        if (slot >= n) slot = 0xFFFFFFFFu;
      }
      // the records go out with lanes 2m and 2m + 1 storing the two halves
      // of one record (that of lane m, then of lane 32 + m): each store
      // instruction touches 32 records instead of 64
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
  __syncthreads();
  // the index runs: s_loc[t] now ends tile t's local range, so the tile of
  // local position q is the number of tiles whose range ends at or before q
  const uint32_t count = static_cast<uint32_t>(end > base ? end - base : 0u);
  for (uint32_t q = threadIdx.x; q < count; q += kBucketThreads) {
    uint32_t t = 0;
#pragma unroll
    for (uint32_t step = kBucketMaxTiles; step != 0u; step >>= 1) {
      if (t + step <= ntiles && s_loc[t + step - 1u] <= q) t += step;
    }
    if (t < ntiles) {
      const uint32_t slot = q + s_d[t];
      if (slot < n) tile_idx[slot] = static_cast<uint32_t>(base) + s_inv[q];
    }
  }
}

// tile_scan: workgroup g scans columns [64g, 64g + 64) of hist over the nblk
// rows, in place (exclusive), and writes the column totals to tile_total.
// Wave r of kScanWaves takes the rows [r*R, (r+1)*R), lane l column
// 64g + l, so every load and store of a wave is 64 consecutive words of one
// row; each lane keeps kScanUnroll loads in flight.
constexpr int kScanWaves = 16;
constexpr uint32_t kScanUnroll = 8;
__global__ __launch_bounds__(kScanWaves * 64) void bucket_colscan_kernel(uint32_t* __restrict__ hist,
                                                                         uint32_t nblk, uint32_t ntiles,
                                                                         uint32_t* __restrict__ tile_total) {
  __shared__ uint32_t s_part[kScanWaves][64];
  const uint32_t lane = threadIdx.x & 63u, r = threadIdx.x >> 6;
  const uint32_t t = blockIdx.x * 64u + lane;
  const uint32_t per = (nblk + kScanWaves - 1u) / kScanWaves;
  const uint32_t w0 = r * per;
  const uint32_t w1 = (w0 + per < nblk) ? w0 + per : nblk;
  const bool live = t < ntiles;
  uint32_t part = 0;
  if (live) {
    for (uint32_t w = w0; w < w1; w += kScanUnroll) {
      uint32_t v[kScanUnroll];
#pragma unroll
      for (uint32_t k = 0; k < kScanUnroll; ++k)
        v[k] = (w + k < w1) ? hist[static_cast<size_t>(w + k) * ntiles + t] : 0u;
#pragma unroll
      for (uint32_t k = 0; k < kScanUnroll; ++k) part += v[k];
    }
  }
  s_part[r][lane] = part;
  __syncthreads();
  uint32_t run = 0, total = 0;
#pragma unroll
  for (uint32_t k = 0; k < static_cast<uint32_t>(kScanWaves); ++k) {
    run += (k < r) ? s_part[k][lane] : 0u;
    total += s_part[k][lane];
  }
  if (live) {
    for (uint32_t w = w0; w < w1; w += kScanUnroll) {
      uint32_t v[kScanUnroll];
#pragma unroll
      for (uint32_t k = 0; k < kScanUnroll; ++k)
        v[k] = (w + k < w1) ? hist[static_cast<size_t>(w + k) * ntiles + t] : 0u;
#pragma unroll
      for (uint32_t k = 0; k < kScanUnroll; ++k) {
        if (w + k < w1) hist[static_cast<size_t>(w + k) * ntiles + t] = run;
        run += v[k];
      }
    }
    if (r == 0) tile_total[t] = total;
  }
}

}  // namespace ugp
