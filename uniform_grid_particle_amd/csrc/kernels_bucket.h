// kernels_bucket.h -- the index build for more particles than the staged
// path takes (n > 2^21) or more cells (keys up to 2^26). Every record moves
// in runs: writing a 32-byte record at a time to scattered places costs
// about three times what whole 128-byte lines cost on MI355X (measured:
// 2^24 records, 790 us scattered one by one, 276 us as randomly placed
// whole lines, 261 us copied), so no pass here scatters single records.
//
// A tile is 2^shift consecutive cell keys (fine tiles, up to 4096, sized so
// a tile holds about 4096 particles on average, as on the staged path); a
// bucket is up to 64 consecutive tiles (2^cshift keys, at most 64 buckets).
//
//   coarse_sort  the staged path's chunk kernel (kernels_staged.h) with
//                buckets for tiles: cell key per particle (celdaDe), each
//                2048-particle chunk counting-sorted by bucket in LDS and
//                written back contiguously, one row {count, prefix} per
//                (chunk, bucket). A chunk's run of one bucket averages
//                2048 / 64 = 32 records.
//   tile_scan    fine_count: the cell keys (celdaDe) of every quarter row
//                block (kRbChunks / 4 chunks of particles) counted per tile;
//                then the column scan of that [quarter x tile] matrix
//                (exclusive, in place), the tile totals and the sums of 64
//                tiles (one bucket each).
//   rebucket     the same workgroups again: each moves its runs in rounds
//                of up to kRbRound particles, sorts a round by tile in LDS
//                and writes every tile's group contiguously at the tile's
//                start plus the row block's offset in it, so the tiles end
//                up contiguous (about 32 records per group). Row block 0
//                also writes one row {count, start} per tile.
//   tile_sort    the staged tile kernel with one contiguous run per tile
//                (kernels_staged.h), as on the staged path's last step.
//
// Against the pages' chain this moves the records three times (into
// buckets, into tiles, into cells) where the pages scatter and gather one
// record per particle; every one of these moves is a run.
#pragma once

#include "common.h"
#include "kernels_staged.h"

namespace ugp {

constexpr uint32_t kBucketMaxTiles = 4096;  // tiles at most
constexpr uint32_t kMaxBuckets = 64;        // buckets at most (coarse_sort LDS bins: <= kStagedMaxTiles)
constexpr uint32_t kMaxFine = 64;           // tiles per bucket at most
constexpr uint32_t kRbChunks = 64;          // chunks per row block
constexpr int kRbThreads = 256;             // fine_count and rebucket workgroups
constexpr uint32_t kRbRound = 2048;         // particles a rebucket round stages in LDS
constexpr uint32_t kRbPer = kRbRound / kRbThreads;  // particles per thread in a round
static_assert(kRbChunks <= 64, "a row block's run table is one wave wide");
constexpr uint32_t kRunTable = 64;  // run table entries (lanes past kRbChunks hold empty runs)
static_assert(kMaxFine <= 64, "a bucket's tiles are one wave wide");

// The run table of row block rb for bucket B: chunks [rb*kRbChunks, ...)
// of the coarse chunk array, s_pre[k] = particles of the runs before chunk
// k of the block, s_src[k] = where chunk k's run starts; returns the block's
// total for the bucket. rows1 holds the coarse rows [chunk x nbuckets].
// Wave 0 does it (one lane per chunk); the caller's barrier follows.
__device__ __forceinline__ void bucket_run_table(const uint2* __restrict__ rows1, uint32_t nchunks,
                                                 uint32_t nbuckets, uint32_t rb, uint32_t B,
                                                 uint32_t* s_pre, uint32_t* s_src, uint32_t* s_total) {
  if (threadIdx.x >= 64) return;
  const uint32_t lane = threadIdx.x;
  const uint32_t c = rb * kRbChunks + lane;
  uint2 r = make_uint2(0u, 0u);
  if (lane < kRbChunks && c < nchunks) r = rows1[static_cast<size_t>(c) * nbuckets + B];
  const uint32_t incl = wave_inclusive_sum(r.x);
  s_pre[lane] = incl - r.x;
  s_src[lane] = c * kChunk + r.y;
  if (lane == 63) *s_total = incl;
}

// The chunk of the block holding the block's p-th particle of the bucket
// (the last chunk whose runs start at or before p; runs in chunk order).
__device__ __forceinline__ uint32_t bucket_run_of(const uint32_t* s_pre, uint32_t p) {
  uint32_t k = 0;
#pragma unroll
  for (uint32_t step = kRunTable / 2; step != 0u; step >>= 1)
    if (s_pre[k + step] <= p) k += step;
  return k;
}

// fine_count: workgroup w counts the cell keys of particles
// [w * kCountPer, (w+1) * kCountPer) per tile into hist[w * ntiles + t]
// (celdaDe read with 16-byte loads, counted in LDS). kCountSub count rows
// make one row block, so the column scan's exclusive prefix at row
// rb * kCountSub is what the row blocks before rb put in each tile.
constexpr int kCountThreads = 1024;
constexpr uint32_t kCountSub = 4;
constexpr uint32_t kCountPer = kRbChunks * kChunk / kCountSub;  // particles per count row
static_assert(kCountPer % (4u * kCountThreads) == 0, "whole 16-byte loads per thread");
__global__ __launch_bounds__(kCountThreads) void bucket_fine_count_kernel(
    const uint32_t* __restrict__ celdaDe, uint32_t n, uint32_t tile_shift, uint32_t ntiles,
    uint32_t* __restrict__ hist) {
  constexpr uint32_t kLoads = kCountPer / (4u * kCountThreads);  // 16-byte loads per thread
  __shared__ uint32_t s_h[kBucketMaxTiles];
  for (uint32_t t = threadIdx.x; t < ntiles; t += kCountThreads) s_h[t] = 0u;
  __syncthreads();
  const uint64_t base = static_cast<uint64_t>(blockIdx.x) * kCountPer;
  const uint64_t end = (base + kCountPer < n) ? base + kCountPer : n;
  // read once here: non-temporal loads (measured on MI355X: Large 811 -> 805 us)
  const uint4* c4 = reinterpret_cast<const uint4*>(celdaDe + base);  // base: a multiple of 4
  const uint32_t quads = static_cast<uint32_t>((end - base) / 4u);
  uint4 v[kLoads];
#pragma unroll
  for (uint32_t k = 0; k < kLoads; ++k) {
    const uint32_t q = k * kCountThreads + threadIdx.x;
    v[k] = (q < quads) ? load_stream(c4 + q) : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (uint32_t k = 0; k < kLoads; ++k) {
    if (k * kCountThreads + threadIdx.x < quads) {
      atomicAdd(&s_h[v[k].x >> tile_shift], 1u);
      atomicAdd(&s_h[v[k].y >> tile_shift], 1u);
      atomicAdd(&s_h[v[k].z >> tile_shift], 1u);
      atomicAdd(&s_h[v[k].w >> tile_shift], 1u);
    }
  }
  for (uint64_t j = base + 4ull * quads + threadIdx.x; j < end; j += kCountThreads)
    atomicAdd(&s_h[celdaDe[j] >> tile_shift], 1u);
  __syncthreads();
  for (uint32_t t = threadIdx.x; t < ntiles; t += kCountThreads)
    hist[static_cast<size_t>(blockIdx.x) * ntiles + t] = s_h[t];
}

// Row block and bucket of rebucket workgroup w. Workgroups are dealt to the
// 8 XCDs round robin; when the buckets split evenly over the XCDs, XCD x
// takes the buckets x, x + 8, ... and walks the row blocks of one bucket in
// order, so the workgroups it runs at one time write neighbouring segments
// of every tile and share the lines at their boundaries in its L2.
__device__ __forceinline__ uint2 rebucket_item(uint32_t w, uint32_t nrb, uint32_t nbuckets) {
  if (nbuckets % 8u != 0u) return make_uint2(w % nrb, w / nrb);
  const uint32_t x = w % 8u, i = w / 8u;
  return make_uint2(i % nrb, x + 8u * (i / nrb));
}

// rebucket: workgroup (rb, B) moves the runs of bucket B in row block rb.
// hist holds the column-scanned count matrix (row rb * kCountSub: what the
// row blocks before rb put in each tile), tile_total the tile totals,
// group_total the sums of 64 consecutive tiles (one bucket each). Each tile's group of a round goes to
// tile_rec/tile_idx at the tile's start plus this row block's offset in the
// tile plus what earlier rounds put there; row block 0 writes
// rows[t] = {tile_total[t], start of tile t}.
__global__ __launch_bounds__(kRbThreads) void bucket_rebucket_kernel(
    const uint2* __restrict__ rows1, uint32_t nchunks, uint32_t nbuckets,
    const uint4* __restrict__ chunk_rec, const uint32_t* __restrict__ chunk_idx, uint32_t nrb,
    uint32_t tile_shift, uint32_t fpb, uint32_t ntiles, const uint32_t* __restrict__ hist,
    const uint32_t* __restrict__ tile_total, const uint32_t* __restrict__ group_total, uint32_t n,
    uint4* __restrict__ tile_rec, uint32_t* __restrict__ tile_idx, uint2* __restrict__ rows) {
  __shared__ uint4 s_rec[2 * kRbRound];
  __shared__ uint32_t s_id[kRbRound];
  __shared__ uint8_t s_f[kRbRound];
  __shared__ uint32_t s_pre[kRunTable], s_src[kRunTable], s_total;
  __shared__ uint32_t s_cnt[kMaxFine], s_off[kMaxFine], s_cur[kMaxFine];
  const uint2 item = rebucket_item(blockIdx.x, nrb, nbuckets);
  const uint32_t rb = item.x, B = item.y;
  bucket_run_table(rows1, nchunks, nbuckets, rb, B, s_pre, s_src, &s_total);
  if (threadIdx.x >= 64 && threadIdx.x < 128) {
    // wave 1: the cursors. Start of the bucket's first tile t0 = the groups
    // of 64 tiles before it plus the tiles of its own group before it; then
    // each tile's start within the bucket
    const uint32_t lane = threadIdx.x - 64;
    const uint32_t t0 = B * fpb;
    const uint32_t g0 = t0 / 64u;
    uint32_t v = (lane < g0) ? group_total[lane] : 0u;
    if (64u * g0 + lane < t0) v += tile_total[64u * g0 + lane];
    const uint32_t bstart = wave_inclusive_sum(v);  // lane 63 holds the sum
    const uint32_t base_all = static_cast<uint32_t>(__shfl(static_cast<int>(bstart), 63));
    const uint32_t t = t0 + lane;
    const uint32_t tot = (lane < fpb && t < ntiles) ? tile_total[t] : 0u;
    const uint32_t start = base_all + wave_inclusive_sum(tot) - tot;
    if (lane < fpb) {
      s_cur[lane] = (t < ntiles) ? start + hist[static_cast<size_t>(rb) * kCountSub * ntiles + t] : 0u;
      if (rb == 0 && t < ntiles) rows[t] = make_uint2(tot, start);
    }
  }
  __syncthreads();
  const uint32_t total = s_total;
  for (uint32_t base = 0; base < total; base += kRbRound) {  // workgroup-uniform
    const uint32_t len = (total - base < kRbRound) ? total - base : kRbRound;
    if (threadIdx.x < kMaxFine) s_cnt[threadIdx.x] = 0u;
    uint32_t w[8][kRbPer], id[kRbPer], fr[kRbPer], ft[kRbPer];
#pragma unroll
    for (uint32_t k = 0; k < kRbPer; ++k) {
      const uint32_t p = base + k * kRbThreads + threadIdx.x;
      const uint32_t q = (p < base + len) ? p : base;  // clamped: loads below are unconditional
      const uint32_t j = bucket_run_of(s_pre, q);
      const uint32_t src = s_src[j] + (q - s_pre[j]);
      const uint32_t word = chunk_idx[src];
      const uint4 a = chunk_rec[static_cast<size_t>(src) * 2u];
      const uint4 b = chunk_rec[static_cast<size_t>(src) * 2u + 1u];
      w[0][k] = a.x; w[1][k] = a.y; w[2][k] = a.z; w[3][k] = a.w;
      w[4][k] = b.x; w[5][k] = b.y; w[6][k] = b.z; w[7][k] = b.w;
      // the particle: its chunk's first index plus the index inside the
      // chunk; its tile in the bucket: the bucket-local cell's high bits
      id[k] = (src & ~(kChunk - 1u)) + (word & ((1u << kIdxBits) - 1u));
      ft[k] = (word >> kIdxBits) >> tile_shift;
    }
    __syncthreads();  // s_cnt zeroed; the previous round's LDS reads are done
#pragma unroll
    for (uint32_t k = 0; k < kRbPer; ++k) {
      const uint32_t p = k * kRbThreads + threadIdx.x;
      const uint32_t f = ft[k];
      fr[k] = (p < len && f < fpb) ? (f << 16) | atomicAdd(&s_cnt[f], 1u) : 0xFFFFFFFFu;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      const uint32_t c = (threadIdx.x < kMaxFine) ? s_cnt[threadIdx.x] : 0u;
      const uint32_t ex = wave_inclusive_sum(c) - c;
      if (threadIdx.x < kMaxFine) s_off[threadIdx.x] = ex;
    }
    __syncthreads();
#pragma unroll
    for (uint32_t k = 0; k < kRbPer; ++k) {
      if (fr[k] == 0xFFFFFFFFu) continue;
      const uint32_t f = fr[k] >> 16;
      const uint32_t o = s_off[f] + (fr[k] & 0xFFFFu);
      s_rec[2 * o] = make_uint4(w[0][k], w[1][k], w[2][k], w[3][k]);
      s_rec[2 * o + 1] = make_uint4(w[4][k], w[5][k], w[6][k], w[7][k]);
      s_id[o] = id[k];
      s_f[o] = static_cast<uint8_t>(f);
    }
    __syncthreads();
    // every tile's group out contiguously: 16-byte halves, consecutive
    // lanes on consecutive halves
    for (uint32_t h = threadIdx.x; h < 2 * len; h += kRbThreads) {
      const uint32_t o = h >> 1, f = s_f[o];
      const uint32_t d = s_cur[f] + (o - s_off[f]);
      if (d < n) tile_rec[static_cast<size_t>(d) * 2u + (h & 1u)] = s_rec[h];
    }
    for (uint32_t o = threadIdx.x; o < len; o += kRbThreads) {
      const uint32_t f = s_f[o];
      const uint32_t d = s_cur[f] + (o - s_off[f]);
      if (d < n) tile_idx[d] = s_id[o];
    }
    __syncthreads();
    if (threadIdx.x < kMaxFine) s_cur[threadIdx.x] += s_cnt[threadIdx.x];
  }
}

// tile_scan: workgroup g scans columns [64g, 64g + 64) of hist over the
// nrows rows, in place (exclusive), and writes the column totals to
// tile_total and their sum to group_total[g]. Wave r of kScanWaves takes the
// rows [r*R, (r+1)*R), lane l column 64g + l, so every load and store of a
// wave is 64 consecutive words of one row; each lane keeps kScanUnroll loads
// in flight.
constexpr int kScanWaves = 16;
constexpr uint32_t kScanUnroll = 8;
__global__ __launch_bounds__(kScanWaves * 64) void bucket_colscan_kernel(uint32_t* __restrict__ hist,
                                                                         uint32_t nrows, uint32_t ntiles,
                                                                         uint32_t* __restrict__ tile_total,
                                                                         uint32_t* __restrict__ group_total) {
  __shared__ uint32_t s_part[kScanWaves][64];
  const uint32_t lane = threadIdx.x & 63u, r = threadIdx.x >> 6;
  const uint32_t t = blockIdx.x * 64u + lane;
  const uint32_t per = (nrows + kScanWaves - 1u) / kScanWaves;
  const uint32_t w0 = r * per;
  const uint32_t w1 = (w0 + per < nrows) ? w0 + per : nrows;
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
  // the group's sum (its 64 tiles) for the rebucket cursors
  if (r == 0) {
    const uint32_t g = wave_inclusive_sum(live ? total : 0u);
    if (lane == 63) group_total[blockIdx.x] = g;
  }
}

}  // namespace ugp
