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
//   tile_scan    fine_count: one workgroup per (row block of kRbChunks
//                chunks, bucket) counts the block's runs of that bucket per
//                tile, from the packed index words alone; then the column
//                scan of that [row block x tile] matrix (exclusive, in
//                place), the tile totals and per-64-tile group totals.
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
  if (lane < kRbChunks) {
    s_pre[lane] = incl - r.x;
    s_src[lane] = c * kChunk + r.y;
  }
  if (lane == 63) *s_total = incl;
}

// The chunk of the block holding the block's p-th particle of the bucket
// (the last chunk whose runs start at or before p; runs in chunk order).
__device__ __forceinline__ uint32_t bucket_run_of(const uint32_t* s_pre, uint32_t p) {
  uint32_t k = 0;
#pragma unroll
  for (uint32_t step = kRbChunks / 2; step != 0u; step >>= 1)
    if (s_pre[k + step] <= p) k += step;
  return k;
}

// fine_count: workgroup (rb, B) = (blockIdx.x, blockIdx.y) counts its runs
// per tile into hist[rb * ntiles + B * fpb + f] (f < fpb tiles in the
// bucket), from the packed index words (bucket-local cell << kIdxBits).
__global__ __launch_bounds__(kRbThreads) void bucket_fine_count_kernel(
    const uint2* __restrict__ rows1, uint32_t nchunks, uint32_t nbuckets,
    const uint32_t* __restrict__ chunk_idx, uint32_t tile_shift, uint32_t fpb, uint32_t ntiles,
    uint32_t* __restrict__ hist) {
  __shared__ uint32_t s_pre[kRbChunks], s_src[kRbChunks], s_total;
  __shared__ uint32_t s_h[kMaxFine];
  const uint32_t rb = blockIdx.x, B = blockIdx.y;
  if (threadIdx.x < kMaxFine) s_h[threadIdx.x] = 0u;
  bucket_run_table(rows1, nchunks, nbuckets, rb, B, s_pre, s_src, &s_total);
  __syncthreads();
  const uint32_t total = s_total;
  constexpr uint32_t kBatch = 8;  // index words per thread in flight
  for (uint32_t p0 = 0; p0 < total; p0 += kRbThreads * kBatch) {
    uint32_t word[kBatch];
#pragma unroll
    for (uint32_t k = 0; k < kBatch; ++k) {
      const uint32_t p = p0 + k * kRbThreads + threadIdx.x;
      word[k] = 0xFFFFFFFFu;
      if (p < total) {
        const uint32_t j = bucket_run_of(s_pre, p);
        word[k] = chunk_idx[s_src[j] + (p - s_pre[j])];
      }
    }
#pragma unroll
    for (uint32_t k = 0; k < kBatch; ++k) {
      if (word[k] == 0xFFFFFFFFu) continue;
      const uint32_t f = (word[k] >> kIdxBits) >> tile_shift;
      if (f < fpb) atomicAdd(&s_h[f], 1u);
    }
  }
  __syncthreads();
  if (threadIdx.x < fpb) {
    const uint32_t t = B * fpb + threadIdx.x;
    if (t < ntiles) hist[static_cast<size_t>(rb) * ntiles + t] = s_h[threadIdx.x];
  }
}

// rebucket: workgroup (rb, B) moves the runs fine_count counted. hist holds
// the column-scanned matrix, tile_total the tile totals, group_total the
// sums of 64 consecutive tiles. Each tile's group of a round goes to
// tile_rec/tile_idx at the tile's start plus this row block's offset in the
// tile plus what earlier rounds put there; row block 0 writes
// rows[t] = {tile_total[t], start of tile t}.
__global__ __launch_bounds__(kRbThreads) void bucket_rebucket_kernel(
    const uint2* __restrict__ rows1, uint32_t nchunks, uint32_t nbuckets,
    const uint4* __restrict__ chunk_rec, const uint32_t* __restrict__ chunk_idx, uint32_t tile_shift,
    uint32_t fpb, uint32_t ntiles, const uint32_t* __restrict__ hist,
    const uint32_t* __restrict__ tile_total, const uint32_t* __restrict__ group_total, uint32_t n,
    uint4* __restrict__ tile_rec, uint32_t* __restrict__ tile_idx, uint2* __restrict__ rows) {
  __shared__ uint4 s_rec[2 * kRbRound];
  __shared__ uint32_t s_id[kRbRound];
  __shared__ uint8_t s_f[kRbRound];
  __shared__ uint32_t s_pre[kRbChunks], s_src[kRbChunks], s_total;
  __shared__ uint32_t s_cnt[kMaxFine], s_off[kMaxFine], s_cur[kMaxFine];
  const uint32_t rb = blockIdx.x, B = blockIdx.y;
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
      s_cur[lane] = (t < ntiles) ? start + hist[static_cast<size_t>(rb) * ntiles + t] : 0u;
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

// tile_scan: workgroup g scans columns [64g, 64g + 64) of hist over the nblk
// rows, in place (exclusive), and writes the column totals to tile_total
// and their sum to group_total[g]. Wave r of kScanWaves takes the rows [r*R, (r+1)*R), lane l column
// 64g + l, so every load and store of a wave is 64 consecutive words of one
// row; each lane keeps kScanUnroll loads in flight.
constexpr int kScanWaves = 16;
constexpr uint32_t kScanUnroll = 8;
__global__ __launch_bounds__(kScanWaves * 64) void bucket_colscan_kernel(uint32_t* __restrict__ hist,
                                                                         uint32_t nblk, uint32_t ntiles,
                                                                         uint32_t* __restrict__ tile_total,
                                                                         uint32_t* __restrict__ group_total) {
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
  // the group's sum (its 64 tiles) for the rebucket cursors
  if (r == 0) {
    const uint32_t g = wave_inclusive_sum(live ? total : 0u);
    if (lane == 63) group_total[blockIdx.x] = g;
  }
}

}  // namespace ugp
