// kernels_staged.h -- the two-kernel index build (up to 2^21 particles on
// grids of up to 2^22 keys; the tile kernel also ends the bucketed path of
// kernels_bucket.h and, alone, builds inputs that fit one tile).
//
// Measured on MI355X: a dependent kernel boundary costs about 2.6 us, a
// device-scope global atomic is a memory-side operation (about 23 G/s for
// the whole chip, whatever the address range), and a random 32-byte record
// access moves a whole 128-byte cache line. So this path has two kernels,
// no global atomics, and moves every record with coalesced accesses,
// reordering through LDS:
//
//   chunk_sort  one workgroup per chunk of particles: cell key per
//               particle (celdaDe), a counting sort of the chunk by tile in
//               LDS (a tile is 2^shift consecutive cells, at most 512 tiles),
//               the chunk written back contiguously in tile order (records
//               and particle indices), and one row {count, exclusive prefix}
//               per tile for the chunk.
//   tile_sort   one workgroup per tile: it reads the chunk rows of its tile
//               (how many of its particles each chunk holds, and where), sums
//               them into its start (the tile start is the number of
//               particles in earlier tiles), expands the runs into a
//               per-particle source map in LDS, loads its particles run by
//               run, counts them into an LDS histogram of its cells
//               (conteos) keeping each particle's rank in its cell, scans
//               the histogram (inicios), and writes ordenado and reordered
//               at start + rank through an LDS staging window so the stores
//               are contiguous. A tile with more particles than the
//               registers hold (8192) is counted by its workgroup (the
//               owner) and scattered in rounds of 4096 shared with every
//               other workgroup through a queue of 64 slots (TileQueue),
//               each round taking places from the slot's per-cell cursors
//               with device atomics; past 64 such tiles, a tile scatters
//               alone in rounds of 8192 from LDS cursors.
//
// The tile kernel is compiled per tile shift (4..14) and per variant:
// records moved or not, overflow diagnostics, stable order, single tile.
//
// The result is the counting sort of the pages: exact histogram, exclusive
// scan with the total in the extra slot, every particle inside its cell's
// range; only the order inside a cell depends on LDS atomic arrival order,
// as with the pages' atomic cursor (page "Construir el índice de la rejilla
// con un prefix sum", section "El orden dentro de la celda"), unless the
// stable variant puts it in particle-index order.
#pragma once

#include "common.h"
#include "kernels_diag.h"

namespace ugp {

constexpr int kChunkItems = 8;                      // particles per chunk_sort thread
constexpr uint32_t kStagedMaxTiles = 512;            // tiles at most on the staged path (chunk_sort LDS bins)
constexpr uint32_t kStagedMaxChunks = 1024;          // chunks at most (one row per chunk in tile_sort)
constexpr int kStagedRegs = 8;                      // particles per tile_sort thread in registers
constexpr uint32_t kShortRun = 64;                  // longest chunk run a thread expands by itself

// Geometry the host uses (chosen by measurement on MI355X, 1M particles on
// 128^3 cells: runs of 8+ records per chunk and tile keep tile_sort's loads
// efficient, 2048-particle chunks let two chunk_sort workgroups share a CU).
constexpr int kChunkThreads = 256;                  // chunk_sort workgroup
constexpr uint32_t kChunk = kChunkThreads * kChunkItems;  // 2048 particles per chunk
// inputs of up to kSmallChunkMaxN particles: 512-particle chunks, so that
// more than a few dozen chunk_sort workgroups share the latency-bound work
constexpr int kSmallChunkThreads = 64;
constexpr uint32_t kSmallChunk = kSmallChunkThreads * kChunkItems;
constexpr uint32_t kSmallChunkMaxN = 1u << 18;
constexpr uint32_t kStagedMinShift = 4;            // at least 16 cells per tile
constexpr uint32_t kStagedMaxShift = 14;            // up to 16384 cells per tile
constexpr uint64_t kStagedTarget = 4096;            // mean particles per tile sought (half the capacity)
constexpr int kCellsThreads = 1024;                 // tile_sort workgroup
constexpr uint32_t kSingleMax = kCellsThreads * kStagedRegs;  // particles one tile kernel workgroup stages
constexpr uint32_t kSingleSplitLog = 6;             // single path: up to 2^6 tiles (no diagnostics, no stable order)
constexpr uint32_t kCellsWin = 2048;                // tile_sort LDS staging window

// Words shared through the tile kernel's queue are written and read with
// device-scope atomic operations, which are coherent across the XCDs'
// separate L2 caches without writing back or invalidating those caches
// (a release or acquire fence at device scope would do both, for every
// line, while other workgroups stream their tiles).
__device__ __forceinline__ uint32_t shared_load(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void shared_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tile t's workgroup index, spreading consecutive tiles over workgroups of
// the same XCD (workgroups are dealt to the 8 XCDs round robin), so tiles
// that read neighbouring runs of each chunk share that XCD's L2 lines.
__device__ __forceinline__ uint32_t tile_of_block(uint32_t b, uint32_t ntiles) {
  if (ntiles % 8 != 0) return b;
  return (b % 8) * (ntiles / 8) + b / 8;
}

// chunk_sort: CT threads, chunk b holds particles [b*chunk, (b+1)*chunk)
// with chunk = CT * kChunkItems.
// rows[b*ntiles + t] = {particles of chunk b in tile t, those in tiles < t}.
// chunk_idx[q] = (tile-local cell << kIdxBits) | index inside the chunk.
// diag, fix_counts, queue_hdr (or nullptr): words the tile kernel
// accumulates into, zeroed here. nt_out (1 on the bucketed path): the input
// is read with non-temporal loads, and the chunk array's write-through stores
// also carry the non-temporal bit.
template <int CT>
__global__ __launch_bounds__(CT) void staged_keys_kernel(
    const uint4* __restrict__ parts, uint32_t n, GridParams g, uint32_t* __restrict__ celdaDe,
    uint2* __restrict__ rows, uint32_t tile_shift, uint32_t ntiles, uint4* __restrict__ chunk_rec,
    uint32_t* __restrict__ chunk_idx, uint32_t* __restrict__ diag, uint32_t* __restrict__ fix_counts,
    uint32_t* __restrict__ queue_hdr, uint32_t nt_out) {
  constexpr int kChunkThreads = CT;
  constexpr uint32_t kChunk = CT * kChunkItems;
  constexpr uint32_t kTilesPerThread = kStagedMaxTiles / CT;  // tile bins per thread
  static_assert(kStagedMaxTiles % CT == 0, "whole tile bins per thread");
  __shared__ uint4 s_rec[2 * kChunk];  // the chunk in tile order
  __shared__ uint32_t s_idx[kChunk];
  __shared__ uint32_t s_hist[kStagedMaxTiles];
  __shared__ uint32_t s_wave[kChunkThreads / 64];

  for (uint32_t t = threadIdx.x; t < kStagedMaxTiles; t += kChunkThreads) s_hist[t] = 0u;
  const uint32_t tile_mask = (1u << tile_shift) - 1u;
  // the overflow diagnostics (when asked for) accumulate in tile_sort
  if (diag != nullptr && blockIdx.x == 0 && threadIdx.x < 2) diag[threadIdx.x] = 0u;
  if (fix_counts != nullptr && blockIdx.x == 0 && threadIdx.x < 2) fix_counts[threadIdx.x] = 0u;  // stable fix-up lists
  if (queue_hdr != nullptr && blockIdx.x == 0)  // shared rounds: claimed slots and ready flags
    for (uint32_t j = threadIdx.x; j < kQueueHeader; j += CT) queue_hdr[j] = 0u;
  static_assert(kChunk <= (1u << kIdxBits), "chunk-local indices fit their field");
  const uint32_t base = blockIdx.x * kChunk;
  // the records stay in registers (scalar arrays, static indices) until
  // they are placed in LDS in tile order. Plain loads on the staged path,
  // non-temporal ones on the bucketed path (nt_out): measured on MI355X,
  // plain loads took Baseline 35.58 -> 35.35 us and Large 804 -> 812 us.
  uint32_t w[8][kChunkItems];
  if (nt_out != 0u) {  // uniform
#pragma unroll
    for (int j = 0; j < kChunkItems; ++j) {
      const uint32_t i = base + j * kChunkThreads + threadIdx.x;
      const size_t ic = (i < n) ? i : n - 1u;  // unconditional loads, clamped index
      const uint4 a = load_stream(parts + ic * 2u);
      const uint4 b = load_stream(parts + ic * 2u + 1u);
      w[0][j] = a.x; w[1][j] = a.y; w[2][j] = a.z; w[3][j] = a.w;
      w[4][j] = b.x; w[5][j] = b.y; w[6][j] = b.z; w[7][j] = b.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kChunkItems; ++j) {
      const uint32_t i = base + j * kChunkThreads + threadIdx.x;
      const size_t ic = (i < n) ? i : n - 1u;  // unconditional loads, clamped index
      const uint4 a = parts[ic * 2u];
      const uint4 b = parts[ic * 2u + 1u];
      w[0][j] = a.x; w[1][j] = a.y; w[2][j] = a.z; w[3][j] = a.w;
      w[4][j] = b.x; w[5][j] = b.y; w[6][j] = b.z; w[7][j] = b.w;
    }
  }
  __syncthreads();  // s_hist zeroed
  // cell keys and tile ranks; the keys go out at once (celdaDe), so those
  // stores drain while the chunk is sorted in LDS (memory operations
  // complete in issue order, so waiting for a record register loaded
  // before them does not wait for them)
  uint32_t cellv[kChunkItems], rank[kChunkItems];
#pragma unroll
  for (int j = 0; j < kChunkItems; ++j) {
    const uint32_t i = base + j * kChunkThreads + threadIdx.x;
    const bool act = i < n;
    const uint32_t c = cell_of(__uint_as_float(w[0][j]), __uint_as_float(w[1][j]),
                               __uint_as_float(w[2][j]), g);
    cellv[j] = act ? c : 0xFFFFFFFFu;
    rank[j] = act ? atomicAdd(&s_hist[c >> tile_shift], 1u) : 0u;
  }
#pragma unroll
  for (int j = 0; j < kChunkItems; ++j)
    if (cellv[j] != 0xFFFFFFFFu) celdaDe[base + j * kChunkThreads + threadIdx.x] = cellv[j];
  __syncthreads();
  // exclusive scan of the tile histogram: kTilesPerThread consecutive bins per thread
  uint32_t cnt[kTilesPerThread], exq[kTilesPerThread];
  uint32_t sum = 0;
#pragma unroll
  for (uint32_t q = 0; q < kTilesPerThread; ++q) {
    const uint32_t t = threadIdx.x * kTilesPerThread + q;
    cnt[q] = (t < ntiles) ? s_hist[t] : 0u;
    sum += cnt[q];
  }
  uint32_t total;
  uint32_t ex = block_exclusive_sum<kChunkThreads>(sum, s_wave, &total);
#pragma unroll
  for (uint32_t q = 0; q < kTilesPerThread; ++q) {
    const uint32_t t = threadIdx.x * kTilesPerThread + q;
    exq[q] = ex;
    if (t < ntiles) s_hist[t] = ex;  // now the first local slot of each tile
    ex += cnt[q];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kChunkItems; ++j) {
    if (cellv[j] != 0xFFFFFFFFu) {
      const uint32_t local = s_hist[cellv[j] >> tile_shift] + rank[j];
      s_rec[2 * local] = make_uint4(w[0][j], w[1][j], w[2][j], w[3][j]);
      s_rec[2 * local + 1] = make_uint4(w[4][j], w[5][j], w[6][j], w[7][j]);
      s_idx[local] = ((cellv[j] & tile_mask) << kIdxBits) | (j * kChunkThreads + threadIdx.x);
    }
  }
  __syncthreads();
  // the chunk in tile order, written contiguously, then the rows. Written
  // through to memory (store_through) by the 2048-particle chunks; the
  // small-chunk variant serves inputs of up to kSmallChunkMaxN particles,
  // whose chunk array (9.4 MB at most) the L2 caches hold, and there plain
  // stores written back at the kernel's end cost less (Sparse 20.56 against
  // 20.86 us written through, Baseline 37.7 against 36.7 us the other way)
  const uint32_t in_chunk = total;  // valid particles of this chunk
  constexpr bool kThrough = CT >= 256;
  uint4* dst = chunk_rec + static_cast<size_t>(base) * 2u;
  uint32_t* dsti = chunk_idx + base;
  if (kThrough) {
    const __amdgpu_buffer_rsrc_t r_rec = output_rsrc(dst, 32u * in_chunk);
    const __amdgpu_buffer_rsrc_t r_idx = output_rsrc(dsti, 4u * in_chunk);
    if (nt_out != 0u) {  // uniform
      for (uint32_t q = threadIdx.x; q < 2 * in_chunk; q += kChunkThreads) store_through_nt(r_rec, 16u * q, s_rec[q]);
      for (uint32_t q = threadIdx.x; q < in_chunk; q += kChunkThreads) store_through_nt(r_idx, 4u * q, s_idx[q]);
    } else {
      for (uint32_t q = threadIdx.x; q < 2 * in_chunk; q += kChunkThreads) store_through(r_rec, 16u * q, s_rec[q]);
      for (uint32_t q = threadIdx.x; q < in_chunk; q += kChunkThreads) store_through(r_idx, 4u * q, s_idx[q]);
    }
  } else {
    for (uint32_t q = threadIdx.x; q < 2 * in_chunk; q += kChunkThreads) dst[q] = s_rec[q];
    for (uint32_t q = threadIdx.x; q < in_chunk; q += kChunkThreads) dsti[q] = s_idx[q];
  }
#pragma unroll
  for (uint32_t q = 0; q < kTilesPerThread; ++q) {
    const uint32_t t = threadIdx.x * kTilesPerThread + q;
    if (t < ntiles) rows[static_cast<size_t>(blockIdx.x) * ntiles + t] = make_uint2(cnt[q], exq[q]);
  }
}

// tile_sort: NT threads; the tile of block b (tile_of_block) owns cells
// [t << SHIFT, (t+1) << SHIFT); WIN records are staged in LDS at a time.
// SINGLE: inputs of at most kSingleMax particles; rows and chunk_idx are
// not read: every workgroup loads the whole input as its one run
// (chunk_rec = the particles, in index order), keeps the particles of its
// own tile, counts those of earlier tiles for its first slot, and writes
// its particles' keys to keys_out (celdaDe), which is not read otherwise.
// With DIAG or STABLE the host launches a single tile: the words those
// variants accumulate into are zeroed here by the workgroup itself.
// MOVE: also write the records (otherwise a separate gather follows).
// DIAG: also fold the tile's histogram into the overflow diagnostics
// (diag[0] max occupancy, diag[1] overflowing insertions over capacity cap;
// both zeroed by the kernel before this one).
// STABLE: every cell lists its particles in ascending index order (page
// "Construir el índice...", section "El orden dentro de la celda"). Each
// particle of a cell of up to kRankSortMax counts the cell's smaller
// particle indices, which is its place in that order, and is staged there.
// A longer cell, and every multi-particle cell of a tile past the staged
// capacity, is written in arrival order and put on one of the fix-up lists;
// a tile holding such a longer cell also copies those arrival-order indices
// to fl.idx() (the whole tile when it is staged, the long cells' ranges when
// it scatters alone, every index when its rounds are shared), which the
// fix-up's long-cell pass reads.
// packed (staged path): chunk_idx words hold the tile-local cell and the
// index inside the chunk (chunk_sort), so no cell key is computed here and
// a particle's index is its chunk's first index plus that field; otherwise
// (bucketed path, single path) a word is the particle index and the cell
// comes from the record's position.
// q (not SINGLE): the shared scatter rounds of tiles past the staged
// capacity (TileQueue), taken by the tile's owner and by every workgroup
// that saw a claimed slot before its own stores. In stable mode the owner
// lists every multi-particle cell of such a tile from its starts, and the
// rounds copy each index to fl.idx() as well.
template <bool MOVE, bool DIAG, bool STABLE, bool SINGLE, uint32_t SHIFT, int NT, uint32_t WIN>
__global__ __launch_bounds__(NT) void staged_cells_kernel(
    const uint2* __restrict__ rows, uint32_t nchunks, uint32_t chunk, uint32_t ntiles, GridParams g,
    uint32_t cells, uint32_t n, const uint4* __restrict__ chunk_rec,
    const uint32_t* __restrict__ chunk_idx, uint32_t* __restrict__ conteos,
    uint32_t* __restrict__ inicios, uint32_t* __restrict__ ordenado, uint4* __restrict__ dst,
    uint32_t cap, uint32_t* __restrict__ diag, FixLists fl, uint32_t* __restrict__ keys_out,
    TileQueue q, uint32_t packed) {
  constexpr uint32_t kTileCells = 1u << SHIFT;
  // cells per thread in the scan (tiles smaller than the workgroup: one
  // cell for each of the first kTileCells threads)
  constexpr uint32_t kPer = (kTileCells >= NT) ? kTileCells / NT : 1u;
  constexpr uint32_t kChunksPerThread = kStagedMaxChunks / NT;
  constexpr uint32_t kStagedCap = NT * kStagedRegs;  // staged tile capacity
  constexpr uint32_t kStagedWin = WIN;
  constexpr uint32_t kRoundPer = kRound / NT;  // particles per thread in a shared round
  constexpr uint32_t kSpinLimit = 1u << 20;  // bound on every wait (each ends in microseconds)
  constexpr uint32_t kIdxMask = (1u << kIdxBits) - 1u;
  static_assert(kTileCells < NT || kTileCells % NT == 0, "whole cells per thread");
  static_assert(SHIFT >= 2, "tiles start on 16-byte boundaries of conteos and inicios");
  static_assert(kStagedMaxChunks % NT == 0, "whole chunk rows per thread");
  static_assert(2 * WIN * 4 >= kStagedCap, "the source map (and, stable, every index) fits in the staging buffer");
  static_assert(kRound % NT == 0 && kRound <= kStagedCap, "a shared round is whole particles per thread");
  static_assert(SHIFT <= 16, "tile-local cells and round ranks share a word");
  static_assert(2 * kStagedMaxChunks <= kQueueRunWords, "a slot's run table holds every chunk's run");
  __shared__ uint32_t s_cnt[kTileCells];
  __shared__ uint32_t s_dst[kStagedMaxChunks];  // tile-local start of each chunk's run
  __shared__ uint32_t s_src[kStagedMaxChunks];  // where that run starts in the chunk array
  __shared__ uint4 s_rec[2 * kStagedWin];
  __shared__ uint32_t s_idx[kStagedWin];
  __shared__ uint32_t s_wave[NT / 64];
  __shared__ uint32_t s_runmax[NT / 64];
  __shared__ uint32_t s_dm[DIAG ? NT / 64 : 1], s_do[DIAG ? NT / 64 : 1];
  // stable: a staged tile has a cell longer than kRankSortMax (0/1); a tile
  // past the capacity counts such cells
  __shared__ uint32_t s_any_long;
  __shared__ uint32_t s_below;  // SINGLE: particles in earlier tiles
  __shared__ uint32_t s_item;   // shared rounds: the item or slot this workgroup took
  __shared__ uint32_t s_list[2];  // stable: the tile's first places on the two fix-up lists

  // one tile holding the whole input: no kernel runs before this one, so the
  // words it would zero are zeroed here, before the first barrier below
  if (SINGLE && threadIdx.x < 2) {
    if (diag != nullptr) diag[threadIdx.x] = 0u;
    if (fl.base != nullptr) fl.base[threadIdx.x] = 0u;
  }
  const bool share = !SINGLE && q.base != nullptr;
  const bool pk = !SINGLE && packed != 0u;
  const uint32_t t = tile_of_block(blockIdx.x, ntiles);
  const uint32_t cell0 = t << SHIFT;
  const uint32_t tc = (cells - cell0 < kTileCells) ? cells - cell0 : kTileCells;

  // chunk runs of this tile (kChunksPerThread consecutive chunks per thread);
  // the tile start is the sum of the chunks' prefixes
  uint2 r[kChunksPerThread];
  uint32_t len_sum = 0, pre_sum = 0;
#pragma unroll
  for (uint32_t k = 0; k < kChunksPerThread; ++k) {
    const uint32_t c = threadIdx.x * kChunksPerThread + k;
    // SINGLE: one run of all n particles
    r[k] = (c < nchunks) ? (SINGLE ? make_uint2(n, 0u) : rows[static_cast<size_t>(c) * ntiles + t]) : make_uint2(0u, 0u);
    len_sum += r[k].x;
    pre_sum += r[k].y;
  }
  uint32_t count;
  // the longest chunk run of the tile (it picks how the source map is built)
  uint32_t my_run = 0;
#pragma unroll
  for (uint32_t k = 0; k < kChunksPerThread; ++k) my_run = (r[k].x > my_run) ? r[k].x : my_run;
  my_run = wave_inclusive_max(my_run);
  if ((threadIdx.x & 63) == 63) s_runmax[threadIdx.x >> 6] = my_run;  // visible after the next barrier
  uint32_t run_dst = block_exclusive_sum<NT>(len_sum, s_wave, &count);
  // the tile's first slot (SINGLE: recomputed below from the particles' keys)
  uint32_t bs = block_sum<NT>(pre_sum, s_wave);
  uint32_t longest_run = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) longest_run = (s_runmax[w] > longest_run) ? s_runmax[w] : longest_run;
  bool short_runs = longest_run <= kShortRun;
#pragma unroll
  for (uint32_t k = 0; k < kChunksPerThread; ++k) {
    const uint32_t c = threadIdx.x * kChunksPerThread + k;
    if (c < nchunks) {
      s_dst[c] = run_dst;
      s_src[c] = c * chunk + r[k].y;  // chunks of `chunk` particles (bucketed, single: one chunk)
    }
    run_dst += r[k].x;
  }
  for (uint32_t j = threadIdx.x; j < kTileCells; j += NT) s_cnt[j] = 0u;
  if (SINGLE && threadIdx.x == 0) s_below = 0u;
  __syncthreads();

  // source map of a window of the tile: s_map[k] = chunk-array position of
  // tile-local particle base + k, for k < len <= kStagedCap (s_map aliases the
  // staging buffer). Runs are laid out in chunk order, so the chunk of a
  // position is the last chunk whose run starts at or before it: every run
  // start (or, for the run covering `base`, position 0) is marked with its
  // chunk number plus one, and an inclusive maximum scan over the window
  // spreads it, whatever the run lengths (a few long runs, as from nearly
  // sorted input). When every run is short (shuffled input) each thread
  // simply expands its own chunk's run instead. The scan contains barriers
  // (the tile-uniform choice keeps them uniform); callers put one before
  // build_map (the previous reads of s_map are done) and one after.
  // r[].x, short_runs, s_dst and s_src describe the tile being mapped (a
  // shared round replaces them with its slot's run table).
  uint32_t* s_map = reinterpret_cast<uint32_t*>(s_rec);
  constexpr uint32_t kMapPer = kStagedCap / NT;  // window entries per thread
  auto build_map = [&](uint32_t base, uint32_t len) __attribute__((always_inline)) {
    const uint32_t end = base + len;
    if (nchunks == 1u) {
      // one run (a tile stored contiguously): the source is its start plus p
      for (uint32_t k = threadIdx.x; k < len; k += NT) s_map[k] = s_src[0] + (base + k);
      return;
    }
    if (short_runs) {
      // every run short: each thread expands the runs of its own chunks
#pragma unroll
      for (uint32_t k = 0; k < kChunksPerThread; ++k) {
        const uint32_t c = threadIdx.x * kChunksPerThread + k;
        if (c < nchunks) {
          const uint32_t d0 = s_dst[c], d1 = d0 + r[k].x;
          const uint32_t lo = (d0 > base) ? d0 : base, hi = (d1 < end) ? d1 : end;
          for (uint32_t j = lo; j < hi; ++j) s_map[j - base] = s_src[c] + (j - d0);
        }
      }
      return;
    }
    const uint32_t m0 = threadIdx.x * kMapPer;
#pragma unroll
    for (uint32_t k = 0; k < kMapPer; ++k) s_map[m0 + k] = 0u;
    __syncthreads();
#pragma unroll
    for (uint32_t k = 0; k < kChunksPerThread; ++k) {
      const uint32_t c = threadIdx.x * kChunksPerThread + k;
      if (c < nchunks && r[k].x > 0u) {
        const uint32_t d0 = s_dst[c], d1 = d0 + r[k].x;
        if (d0 < end && d1 > base) s_map[(d0 > base) ? d0 - base : 0u] = c + 1u;
      }
    }
    __syncthreads();
    uint32_t mark[kMapPer];
    uint32_t run = 0;
#pragma unroll
    for (uint32_t k = 0; k < kMapPer; ++k) {
      mark[k] = s_map[m0 + k];
      run = (mark[k] > run) ? mark[k] : run;
    }
    uint32_t cur = block_exclusive_max<NT>(run, s_wave);
#pragma unroll
    for (uint32_t k = 0; k < kMapPer; ++k) {
      cur = (mark[k] > cur) ? mark[k] : cur;
      const uint32_t pos = base + m0 + k;
      if (m0 + k < len && cur > 0u) s_map[m0 + k] = s_src[cur - 1u] + (pos - s_dst[cur - 1u]);
    }
  };

  // a particle's index from its chunk-array position and index word
  auto index_of = [&](uint32_t src, uint32_t word) __attribute__((always_inline)) -> uint32_t {
    return pk ? (src & ~(chunk - 1u)) + (word & kIdxMask) : word;
  };

  // exclusive scan in LDS: kPer consecutive cells per thread, then the
  // block scan of the per-thread sums; s_cnt becomes the tile-local starts
  // (cells past tc count 0, so their start is the tile total)
  auto scan_tile = [&]() __attribute__((always_inline)) -> uint32_t {
    const uint32_t j0 = threadIdx.x * kPer;
    const bool scans = j0 < kTileCells;
    uint32_t sum = 0;
    if (scans) {
#pragma unroll 4
      for (uint32_t k = 0; k < kPer; ++k) sum += s_cnt[j0 + k];
    }
    uint32_t tot;
    uint32_t run = block_exclusive_sum<NT>(sum, s_wave, &tot);
    if (scans) {
#pragma unroll 4
      for (uint32_t k = 0; k < kPer; ++k) {
        const uint32_t v = s_cnt[j0 + k];
        s_cnt[j0 + k] = run;
        run += v;
      }
    }
    __syncthreads();
    return tot;
  };

  // conteos and inicios out, from the starts: a cell's count is the next
  // start minus its own. Lane-contiguous 16-byte stores (tiles start at
  // multiples of 16 cells), written through to memory (store_through). DIAG:
  // the same counts feed the overflow diagnostics (one more barrier, after
  // which thread 0 publishes).
  auto write_counts_starts = [&](uint32_t tot) __attribute__((always_inline)) {
    const uint4* s_cnt4 = reinterpret_cast<const uint4*>(s_cnt);
    const uint32_t tc4 = tc / 4;
    const __amdgpu_buffer_rsrc_t r_conteos = output_rsrc(conteos + cell0, 16u * tc4);
    const __amdgpu_buffer_rsrc_t r_inicios = output_rsrc(inicios + cell0, 16u * tc4);
    uint32_t dmax = 0, dover = 0;
    for (uint32_t k = threadIdx.x; k < tc4; k += NT) {
      const uint4 v = s_cnt4[k];
      const uint32_t next = (4 * k + 4 < kTileCells) ? s_cnt[4 * k + 4] : tot;
      const uint4 c = make_uint4(v.y - v.x, v.z - v.y, v.w - v.z, next - v.w);
      store_through(r_conteos, 16u * k, c);
      store_through(r_inicios, 16u * k, make_uint4(bs + v.x, bs + v.y, bs + v.z, bs + v.w));
      if (DIAG) {
        const uint32_t a = (c.x > c.y) ? c.x : c.y;
        const uint32_t b = (c.z > c.w) ? c.z : c.w;
        dmax = (a > dmax) ? a : dmax;
        dmax = (b > dmax) ? b : dmax;
        dover += overflow_of(c.x, cap) + overflow_of(c.y, cap) + overflow_of(c.z, cap) + overflow_of(c.w, cap);
      }
    }
    for (uint32_t j = 4 * tc4 + threadIdx.x; j < tc; j += NT) {
      const uint32_t next = (j + 1 < kTileCells) ? s_cnt[j + 1] : tot;
      const uint32_t c = next - s_cnt[j];
      conteos[cell0 + j] = c;
      inicios[cell0 + j] = bs + s_cnt[j];
      if (DIAG) {
        dmax = (c > dmax) ? c : dmax;
        dover += overflow_of(c, cap);
      }
    }
    if (t == ntiles - 1 && threadIdx.x == 0) inicios[cells] = bs + tot;
    if (DIAG) {
      dmax = wave_max_u32(dmax);
      dover = wave_add_u32(dover);
      if ((threadIdx.x & 63) == 0) {
        s_dm[threadIdx.x >> 6] = dmax;
        s_do[threadIdx.x >> 6] = dover;
      }
      __syncthreads();
      publish_diag<NT>(s_dm, s_do, diag);
    }
  };

  // Stable mode: puts the tile's cells of min_len or more particles
  // (len_of(j) for tile-local cell j) on the short or long fix-up list, with
  // one block scan of the per-thread counts and one global atomic per list
  // for the whole tile (each thread takes kPer consecutive cells, so the
  // list holds them in cell order). Contains barriers: call it uniformly.
  auto list_cells_tile = [&](uint32_t min_len, auto len_of) __attribute__((always_inline)) {
    static_assert(kTileCells < (1u << 16), "a tile's list counts fit a half-word");
    const uint32_t j0 = threadIdx.x * kPer;
    uint32_t len[kPer];
    uint32_t ns = 0, nl = 0;
#pragma unroll
    for (uint32_t k = 0; k < kPer; ++k) {
      len[k] = (j0 + k < tc) ? len_of(j0 + k) : 0u;
      const bool listed = len[k] >= min_len;
      ns += (listed && len[k] <= kRankSortMax) ? 1u : 0u;
      nl += (listed && len[k] > kRankSortMax) ? 1u : 0u;
    }
    uint32_t total;
    const uint32_t ex = block_exclusive_sum<NT>(ns | (nl << 16), s_wave, &total);
    if (threadIdx.x == 0) {
      s_list[0] = (total & 0xFFFFu) ? atomicAdd(&fl.base[0], total & 0xFFFFu) : 0u;
      s_list[1] = (total >> 16) ? atomicAdd(&fl.base[1], total >> 16) : 0u;
    }
    __syncthreads();
    uint32_t fs = s_list[0] + (ex & 0xFFFFu), fo = s_list[1] + (ex >> 16);
#pragma unroll
    for (uint32_t k = 0; k < kPer; ++k) {
      if (len[k] < min_len) continue;
      if (len[k] <= kRankSortMax) {
        if (fs < fl.fix_cap) fl.fix()[fs] = cell0 + j0 + k;
        ++fs;
      } else {
        if (fo < fl.long_cap) fl.lng()[fo] = cell0 + j0 + k;
        ++fo;
      }
    }
    __syncthreads();  // s_list is read before it is used again
  };

  // One shared scatter round: positions [base, base + len) of a shared
  // tile's own order (its sources from the source list, or rebuilt from the
  // slot's run table), counted per cell in LDS (rank = the value the LDS
  // atomic returns); every cell the round touches takes a block of places
  // from the slot's cursor with one atomic, and every particle goes to its
  // cell's block plus its rank.
  auto scatter_round = [&](uint32_t slot, uint32_t round, uint32_t wbs, uint32_t wcount,
                           uint32_t wtile, bool by_runs) __attribute__((always_inline)) {
    const uint32_t base = round * kRound;
    if (base >= wcount) return;  // uniform
    const uint32_t len = (wcount - base < kRound) ? wcount - base : kRound;
    const uint32_t rcell0 = wtile << SHIFT;
    const uint32_t rtc = (cells - rcell0 < kTileCells) ? cells - rcell0 : kTileCells;
    uint32_t* cur = q.cursors(slot);
    __syncthreads();  // the previous use of s_cnt (and of s_dst, s_src, s_map) is over
    for (uint32_t j = threadIdx.x; j < kTileCells; j += NT) s_cnt[j] = 0u;
    uint32_t src[kRoundPer], word[kRoundPer], lr[kRoundPer], v[8][kRoundPer];
    if (by_runs) {  // uniform
      // the slot's run table replaces this workgroup's own (its tile is
      // done): every run is short, so each thread expands its own chunk's
      // run over the round's window
      const uint32_t* rt = q.runs(slot);
#pragma unroll
      for (uint32_t k = 0; k < kChunksPerThread; ++k) {
        const uint32_t c = threadIdx.x * kChunksPerThread + k;
        if (c < nchunks) {
          s_dst[c] = shared_load(rt + c);
          s_src[c] = shared_load(rt + kStagedMaxChunks + c);
        }
      }
      __syncthreads();
#pragma unroll
      for (uint32_t k = 0; k < kChunksPerThread; ++k) {
        const uint32_t c = threadIdx.x * kChunksPerThread + k;
        const uint32_t d0 = (c < nchunks) ? s_dst[c] : wcount;
        const uint32_t d1 = (c + 1u < nchunks) ? s_dst[c + 1u] : wcount;
        r[k].x = (d1 > d0) ? d1 - d0 : 0u;
      }
      short_runs = true;
      build_map(base, len);
      __syncthreads();
#pragma unroll
      for (uint32_t k = 0; k < kRoundPer; ++k) {
        const uint32_t j = threadIdx.x + k * NT;
        const uint32_t m = (j < len) ? s_map[j] : 0u;
        src[k] = (m < n) ? m : n - 1u;  // n >= 1: a tile holds particles
      }
    } else {
#pragma unroll
      for (uint32_t k = 0; k < kRoundPer; ++k) {
        const uint32_t j = threadIdx.x + k * NT;
        const size_t pos = static_cast<size_t>(wbs) + base + j;
        const uint32_t m = (j < len && pos < n) ? shared_load(q.sources + pos) : 0u;
        src[k] = (m < n) ? m : n - 1u;  // n >= 1: a tile holds particles
      }
    }
#pragma unroll
    for (uint32_t k = 0; k < kRoundPer; ++k) word[k] = chunk_idx[src[k]];
#pragma unroll
    for (uint32_t k = 0; k < kRoundPer; ++k) {
      const uint4 a = (MOVE || !pk) ? chunk_rec[static_cast<size_t>(src[k]) * 2u] : make_uint4(0u, 0u, 0u, 0u);
      const uint4 b = MOVE ? chunk_rec[static_cast<size_t>(src[k]) * 2u + 1u] : make_uint4(0u, 0u, 0u, 0u);
      v[0][k] = a.x; v[1][k] = a.y; v[2][k] = a.z; v[3][k] = a.w;
      v[4][k] = b.x; v[5][k] = b.y; v[6][k] = b.z; v[7][k] = b.w;
    }
    __syncthreads();  // s_cnt is zero
#pragma unroll
    for (uint32_t k = 0; k < kRoundPer; ++k) {
      const uint32_t j = threadIdx.x + k * NT;
      const uint32_t loc = pk ? word[k] >> kIdxBits
                              : cell_of(__uint_as_float(v[0][k]), __uint_as_float(v[1][k]),
                                        __uint_as_float(v[2][k]), g) - rcell0;
      lr[k] = (j < len && loc < rtc) ? (loc << 16) | atomicAdd(&s_cnt[loc], 1u) : 0xFFFFFFFFu;
    }
    __syncthreads();
    {
      // the block of places this round takes in each cell it touches: the
      // atomics of a batch of 4 cells per thread in flight together
      constexpr uint32_t kCellIter = (kTileCells + NT - 1) / NT;
      constexpr uint32_t kBatch = (kCellIter < 4u) ? kCellIter : 4u;
#pragma unroll 1
      for (uint32_t k0 = 0; k0 < kCellIter; k0 += kBatch) {
        uint32_t cnt[kBatch], at[kBatch];
#pragma unroll
        for (uint32_t k = 0; k < kBatch; ++k) {
          const uint32_t j = threadIdx.x + (k0 + k) * NT;
          cnt[k] = (j < rtc) ? s_cnt[j] : 0u;
          at[k] = (cnt[k] != 0u) ? atomicAdd(&cur[j], cnt[k]) : 0u;
        }
#pragma unroll
        for (uint32_t k = 0; k < kBatch; ++k)
          if (cnt[k] != 0u) s_cnt[threadIdx.x + (k0 + k) * NT] = at[k];
      }
    }
    __syncthreads();
#pragma unroll
    for (uint32_t k = 0; k < kRoundPer; ++k) {
      if (lr[k] == 0xFFFFFFFFu) continue;
      const size_t out = static_cast<size_t>(wbs) + s_cnt[lr[k] >> 16] + (lr[k] & 0xFFFFu);
      if (out < n) {
        const uint32_t id = index_of(src[k], word[k]);
        ordenado[out] = id;
        // stable: every cell of a shared tile is listed for the fix-up, and
        // its long cells read their arrival order from this copy
        if (STABLE) fl.idx()[out] = id;
        if (MOVE) {
          dst[out * 2u] = make_uint4(v[0][k], v[1][k], v[2][k], v[3][k]);
          dst[out * 2u + 1u] = make_uint4(v[4][k], v[5][k], v[6][k], v[7][k]);
        }
      }
    }
  };

  // Takes rounds of the claimed slots until every slot is ready and its
  // ticket has run past its rounds. Wave 0 reads every slot's ready flag,
  // ticket and round count at once (one lane per slot), picks the first
  // slot with rounds left at or after `first` (so that workgroups spread
  // over the slots) and takes a round from its ticket; a slot not ready yet
  // counts as having rounds and is waited for: its owner claimed it, so it
  // is running, and it marks it ready without waiting.
  auto help = [&](uint32_t first) __attribute__((always_inline)) {
    for (;;) {
      __syncthreads();  // every thread has read the previous pick
      if (threadIdx.x < 64) {
        const uint32_t lane = threadIdx.x;
        uint32_t got = 0xFFFFFFFFu, slot = 0, wbs = 0, wcount = 0, wtile = 0;
        for (uint32_t spin = 0; spin < kSpinLimit; ++spin) {
          const uint32_t claimed = shared_load(q.hdr());
          const uint32_t nslots = (claimed < kMaxSlots) ? claimed : kMaxSlots;
          bool ready = false, left = false;
          if (lane < nslots) {
            ready = shared_load(q.hdr() + kReadyWord + lane) != 0u;
            left = !ready || shared_load(q.hdr() + kTicketWord + lane) < shared_load(q.hdr() + kRoundsWord + lane);
          }
          const uint64_t mleft = __ballot(left);
          if (mleft == 0ull) break;  // every slot ready and exhausted
          const uint64_t mready = __ballot(left && ready);
          if (mready == 0ull) {  // rounds remain only in slots not ready yet
            __builtin_amdgcn_s_sleep(2);
            continue;
          }
          // the first ready slot with rounds left at or after `first` (cyclically)
          const uint32_t sh = first % 64u;
          const uint64_t rot = (mready >> sh) | (sh ? (mready << (64u - sh)) : 0ull);
          const uint32_t pick = (static_cast<uint32_t>(__builtin_ctzll(rot)) + sh) % 64u;
          uint32_t r = 0xFFFFFFFFu, nr = 0u, b0 = 0u, c0 = 0u, t0 = 0u;
          if (lane == pick) {
            r = atomicAdd(q.hdr() + kTicketWord + pick, 1u);
            nr = shared_load(q.hdr() + kRoundsWord + pick);
            b0 = shared_load(q.hdr() + kStartWord + pick);
            c0 = shared_load(q.hdr() + kCountWord + pick);
            t0 = shared_load(q.hdr() + kTileWord + pick);
          }
          r = static_cast<uint32_t>(__shfl(static_cast<int>(r), static_cast<int>(pick)));
          nr = static_cast<uint32_t>(__shfl(static_cast<int>(nr), static_cast<int>(pick)));
          if (r < nr) {
            got = r;
            slot = pick;
            wbs = static_cast<uint32_t>(__shfl(static_cast<int>(b0), static_cast<int>(pick)));
            wcount = static_cast<uint32_t>(__shfl(static_cast<int>(c0), static_cast<int>(pick)));
            wtile = static_cast<uint32_t>(__shfl(static_cast<int>(t0), static_cast<int>(pick)));
            break;
          }
        }
        if (lane == 0) {  // s_dst and s_src are free once the workgroup's own tile is done
          s_item = got;
          s_dst[0] = wbs;
          s_src[0] = wcount;
          s_dst[1] = slot;
          s_src[1] = wtile;
        }
      }
      __syncthreads();
      const uint32_t round = s_item, wbs = s_dst[0], wcount = s_src[0], slot = s_dst[1];
      const uint32_t wtile = s_src[1] & ~kRunTableBit;
      const bool by_runs = (s_src[1] & kRunTableBit) != 0u;
      if (round == 0xFFFFFFFFu) return;  // uniform
      if (wtile < ntiles && wcount <= n && wbs <= n - wcount)  // uniform checks keep it in bounds
        scatter_round(slot, round, wbs, wcount, wtile, by_runs);
    }
  };

  if (count <= kStagedCap) {
    // records held in registers as scalar arrays (static indices); lr packs
    // a particle's tile-local cell (high half) and its rank in that cell
    // (low half, < kStagedCap), all ones when the lane holds no particle.
    // The two branches share nothing live, so these registers are not
    // reserved while a tile past the capacity runs.
    uint32_t w[8][kStagedRegs], idx[kStagedRegs], lr[kStagedRegs];
#pragma unroll
    for (int k = 0; k < kStagedRegs; ++k) lr[k] = 0xFFFFFFFFu;
    build_map(0u, count);  // s_dst, s_src: visible since the barrier above
    __syncthreads();
    if (count > 0) {  // count == 0: no valid source to clamp the idle lanes to
      uint32_t src[kStagedRegs];
#pragma unroll
      for (int k = 0; k < kStagedRegs; ++k) {
        const uint32_t p = threadIdx.x + k * NT;
        src[k] = s_map[p < count ? p : 0u];  // clamped: loads below are unconditional
      }
      // index words first, then the records: with packed words the count
      // below needs only the words (loads complete in issue order), so it
      // runs while the records are still on their way
#pragma unroll
      for (int k = 0; k < kStagedRegs; ++k) idx[k] = SINGLE ? src[k] : chunk_idx[src[k]];  // SINGLE: the input itself
#pragma unroll
      for (int k = 0; k < kStagedRegs; ++k) {
        const uint4 a = (MOVE || !pk) ? chunk_rec[static_cast<size_t>(src[k]) * 2u] : make_uint4(0u, 0u, 0u, 0u);
        const uint4 b = MOVE ? chunk_rec[static_cast<size_t>(src[k]) * 2u + 1u] : make_uint4(0u, 0u, 0u, 0u);
        w[0][k] = a.x; w[1][k] = a.y; w[2][k] = a.z; w[3][k] = a.w;
        w[4][k] = b.x; w[5][k] = b.y; w[6][k] = b.z; w[7][k] = b.w;
      }
      // count each particle and keep its rank: its slot is later the
      // cell's start plus that rank
#pragma unroll
      for (int k = 0; k < kStagedRegs; ++k) {
        const uint32_t p = threadIdx.x + k * NT;
        uint32_t loc, key = 0;
        if (pk) {
          loc = idx[k] >> kIdxBits;
          idx[k] = index_of(src[k], idx[k]);
        } else {
          key = cell_of(__uint_as_float(w[0][k]), __uint_as_float(w[1][k]), __uint_as_float(w[2][k]), g);
          loc = key - cell0;
        }
        if (p < count && loc < tc) lr[k] = (loc << 16) | atomicAdd(&s_cnt[loc], 1u);
        if (SINGLE) {  // particles of earlier tiles, one LDS atomic per wave
          const uint64_t m = __ballot(p < count && key < cell0);
          if ((threadIdx.x & 63) == 0 && m != 0ull) atomicAdd(&s_below, static_cast<uint32_t>(__popcll(m)));
        }
      }
      // every record load of this thread has landed: the compiler then needs
      // no wait before using those registers after the stores below (one
      // counter tracks loads and stores alike)
      __builtin_amdgcn_s_waitcnt(kWaitLoadsAndStores);
      if (SINGLE) {
#pragma unroll
        for (int k = 0; k < kStagedRegs; ++k)
          if (lr[k] != 0xFFFFFFFFu) keys_out[idx[k]] = cell0 + (lr[k] >> 16);
      }
    }
    __syncthreads();
    // SINGLE: every workgroup read the whole input; its tile starts after the
    // particles of the tiles before it
    if (SINGLE) bs = s_below;
    // slots claimed so far (owners claim theirs right after reading their
    // rows), read before this tile's stores and kept in s_item, which is
    // unused until the tail: after the stores the workgroup helps only when
    // some slot was claimed (a load used after the stores waits for them)
    if (share && threadIdx.x == 0) s_item = shared_load(q.hdr());
    const uint32_t tot = scan_tile();
    write_counts_starts(tot);  // overlaps the placement below
    uint32_t slot[kStagedRegs];
#pragma unroll
    for (int k = 0; k < kStagedRegs; ++k)
      slot[k] = (lr[k] != 0xFFFFFFFFu) ? s_cnt[lr[k] >> 16] + (lr[k] & 0xFFFFu) : 0xFFFFFFFFu;
    bool any_long = false;  // stable: the tile's indices also go to fl.idx()
    if (STABLE) {
      // every index at its arrival slot (the source map is dead: s_rec is
      // free); then each particle of a cell of up to kRankSortMax counts
      // the cell's smaller indices (distinct), which is its place in index
      // order. A longer cell keeps the arrival order and is listed.
      uint32_t* s_all = reinterpret_cast<uint32_t*>(s_rec);
#pragma unroll
      for (int k = 0; k < kStagedRegs; ++k)
        if (slot[k] != 0xFFFFFFFFu) s_all[slot[k]] = idx[k];
      if (threadIdx.x == 0) s_any_long = 0u;
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kStagedRegs; ++k) {
        if (slot[k] != 0xFFFFFFFFu) {
          const uint32_t loc = lr[k] >> 16;
          const uint32_t a = s_cnt[loc];
          const uint32_t e = (loc + 1u < kTileCells) ? s_cnt[loc + 1u] : tot;
          if (e - a <= kRankSortMax) {
            uint32_t pos = a;
            for (uint32_t j = a; j < e; ++j) pos += (s_all[j] < idx[k]) ? 1u : 0u;
            slot[k] = pos;
          } else {
            s_any_long = 1u;
          }
        }
      }
      __syncthreads();  // every rank counted before the window loop reuses s_rec
      any_long = s_any_long != 0u;
      if (any_long)  // tile-uniform; s_cnt holds the starts
        list_cells_tile(kRankSortMax + 1u,
                        [&](uint32_t j) { return ((j + 1u < kTileCells) ? s_cnt[j + 1u] : tot) - s_cnt[j]; });
    }
    // The staged path's stores: ordenado and the records leave a window at a
    // time, contiguously; the records with the non-temporal hint, which
    // measured on MI355X took Baseline 36.5 -> 35.8 us and Large 847 -> 836
    // us (Sparse and Contention unchanged), while the same hint on ordenado,
    // on the shared rounds' scattered stores or on the loads of the chunk
    // array, and the records written through to memory, were all slower.
    for (uint32_t w0 = 0; w0 < tot; w0 += kStagedWin) {  // tile-uniform
      const uint32_t wn = (tot - w0 < kStagedWin) ? tot - w0 : kStagedWin;
#pragma unroll
      for (int k = 0; k < kStagedRegs; ++k) {
        const uint32_t o = slot[k] - w0;
        if (slot[k] != 0xFFFFFFFFu && o < wn) {
          if (MOVE) {
            s_rec[2 * o] = make_uint4(w[0][k], w[1][k], w[2][k], w[3][k]);
            s_rec[2 * o + 1] = make_uint4(w[4][k], w[5][k], w[6][k], w[7][k]);
          }
          s_idx[o] = idx[k];
        }
      }
      __syncthreads();
      const size_t out0 = static_cast<size_t>(bs) + w0;
      for (uint32_t k = threadIdx.x; k < wn; k += NT) {
        if (out0 + k < n) {
          ordenado[out0 + k] = s_idx[k];
          if (STABLE && any_long) fl.idx()[out0 + k] = s_idx[k];
        }
      }
      if (MOVE) {
        for (uint32_t k = threadIdx.x; k < 2 * wn; k += NT)
          if (out0 * 2u + k < 2ull * n) store_stream(dst + out0 * 2u + k, s_rec[k]);
      }
      __syncthreads();
    }
    if (share && s_item != 0u) help(blockIdx.x);  // uniform: written before the barriers above
  } else {
    // a tile past the staged capacity (count > kStagedCap > 0): claim a
    // slot now, so that tiles still loading see it
    uint32_t sidx = kMaxSlots;
    if (share) {
      if (threadIdx.x == 0) s_item = atomicAdd(q.hdr(), 1u);
      __syncthreads();
      sidx = s_item;
    }
    const bool shared = sidx < kMaxSlots;  // uniform
    // every run short (shuffled input): one pass, each thread counting its
    // own chunk's run (one 16-byte load per four words, all in flight
    // together), and the rounds rebuild their sources from the run table
    const bool by_runs = shared && pk && short_runs && nchunks > 1u;  // uniform
    if (by_runs) {
      constexpr uint32_t kRunLoads = (kShortRun + 6u) / 4u;  // 16-byte loads covering a run of kShortRun
      static_assert(kChunksPerThread == 1, "one chunk run per thread");
      const uint32_t c = threadIdx.x;
      const uint32_t rl = (c < nchunks) ? r[0].x : 0u;  // <= kShortRun
      const uint32_t a = c * chunk + r[0].y;            // the run's first word
      const uint32_t a4 = a & ~3u;
      uint4 wv[kRunLoads];
#pragma unroll
      for (uint32_t m = 0; m < kRunLoads; ++m)
        wv[m] = (rl != 0u && a4 + 4u * m < a + rl) ? reinterpret_cast<const uint4*>(chunk_idx)[a4 / 4u + m]
                                                  : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (uint32_t m = 0; m < kRunLoads; ++m) {
        const uint32_t w0 = a4 + 4u * m;
        const uint32_t e[4] = {wv[m].x, wv[m].y, wv[m].z, wv[m].w};
#pragma unroll
        for (uint32_t i = 0; i < 4; ++i) {
          const uint32_t w = w0 + i;
          const uint32_t loc = e[i] >> kIdxBits;
          if (w >= a && w < a + rl && loc < tc) atomicAdd(&s_cnt[loc], 1u);
        }
      }
    } else {
    // the count goes in rounds of kStagedCap particles (kStagedRegs per thread), each
    // with the source map of its window and its loads in flight together;
    // packed index words give the cells directly, else the positions are
    // read. Shared: the sources go to the source list as well.
    for (uint32_t base = 0; base < count; base += kStagedCap) {
      const uint32_t len = (count - base < kStagedCap) ? count - base : kStagedCap;
      __syncthreads();  // the previous round's map reads are done
      build_map(base, len);
      __syncthreads();
      uint32_t src[kStagedRegs], loc[kStagedRegs];
#pragma unroll
      for (int k = 0; k < kStagedRegs; ++k) {
        const uint32_t p = threadIdx.x + k * NT;
        src[k] = s_map[p < len ? p : 0u];  // clamped: loads below are unconditional
      }
      if (pk) {
#pragma unroll
        for (int k = 0; k < kStagedRegs; ++k) loc[k] = chunk_idx[src[k]] >> kIdxBits;
      } else {
        float px[kStagedRegs], py[kStagedRegs], pz[kStagedRegs];
#pragma unroll
        for (int k = 0; k < kStagedRegs; ++k) {
          const uint4 a = chunk_rec[static_cast<size_t>(src[k]) * 2u];
          px[k] = __uint_as_float(a.x);
          py[k] = __uint_as_float(a.y);
          pz[k] = __uint_as_float(a.z);
        }
#pragma unroll
        for (int k = 0; k < kStagedRegs; ++k) loc[k] = cell_of(px[k], py[k], pz[k], g) - cell0;
      }
#pragma unroll
      for (int k = 0; k < kStagedRegs; ++k) {
        const uint32_t p = base + threadIdx.x + k * NT;
        if (p < count && loc[k] < tc) atomicAdd(&s_cnt[loc[k]], 1u);
      }
      if (shared) {  // after the loads: they complete in issue order, so these stores do not delay them
#pragma unroll
        for (int k = 0; k < kStagedRegs; ++k) {
          const uint32_t p = threadIdx.x + k * NT;
          const uint32_t pos = bs + base + p;  // < n when p < len
          if (p < len) shared_store(q.sources + pos, src[k]);
        }
      }
    }
    }
    __syncthreads();
    const uint32_t tot = scan_tile();
    if (shared) {
      // the cursors (tile-local starts) and the header words go out with
      // device-coherent stores, all complete before the slot is marked
      // ready (each wave waits for its own, then the barrier); conteos and
      // inicios follow
      uint32_t* curs = q.cursors(sidx);
      for (uint32_t j = threadIdx.x; j < tc; j += NT) shared_store(curs + j, s_cnt[j]);
      if (by_runs) {  // the run table: tile-local starts, then chunk-array starts
        uint32_t* rt = q.runs(sidx);
        for (uint32_t c = threadIdx.x; c < nchunks; c += NT) {
          shared_store(rt + c, s_dst[c]);
          shared_store(rt + kStagedMaxChunks + c, s_src[c]);
        }
      }
      if (threadIdx.x == 0) {
        shared_store(q.hdr() + kRoundsWord + sidx, (count + kRound - 1u) / kRound);
        shared_store(q.hdr() + kStartWord + sidx, bs);
        shared_store(q.hdr() + kCountWord + sidx, count);
        shared_store(q.hdr() + kTileWord + sidx, t | (by_runs ? kRunTableBit : 0u));
      }
      __builtin_amdgcn_s_waitcnt(kWaitLoadsAndStores);
      __syncthreads();
      if (threadIdx.x == 0) shared_store(q.hdr() + kReadyWord + sidx, 1u);
    }
    write_counts_starts(tot);
    if (STABLE && shared) {
      // the rounds take slots in arrival order: every cell of two or more
      // is listed now, from the starts (the rounds reuse s_cnt), and the
      // rounds themselves copy every index to fl.idx()
      __syncthreads();  // s_cnt holds the starts (write_counts_starts read them too)
      list_cells_tile(2u, [&](uint32_t j) { return ((j + 1u < kTileCells) ? s_cnt[j + 1u] : tot) - s_cnt[j]; });
    }
    __syncthreads();  // every start read before the cursors advance
    if (shared) help(sidx);
    if (!shared) {
      // alone: the same rounds again, each particle taking its slot from its
      // cell's cursor and written there directly (the tile's output range is
      // small enough that partial lines merge in L2)
      constexpr int kOver = kStagedRegs;
      for (uint32_t base = 0; base < count; base += NT * kOver) {
        const uint32_t len = (count - base < NT * kOver) ? count - base : NT * kOver;
        __syncthreads();  // the previous round's map reads are done
        build_map(base, len);
        __syncthreads();
        uint32_t src[kOver], id[kOver], v[8][kOver];
#pragma unroll
        for (int k = 0; k < kOver; ++k) {
          const uint32_t p = threadIdx.x + k * NT;
          src[k] = s_map[p < len ? p : 0u];
        }
#pragma unroll
        for (int k = 0; k < kOver; ++k) {
          const uint4 a = (MOVE || !pk) ? chunk_rec[static_cast<size_t>(src[k]) * 2u] : make_uint4(0u, 0u, 0u, 0u);
          const uint4 b = MOVE ? chunk_rec[static_cast<size_t>(src[k]) * 2u + 1u] : make_uint4(0u, 0u, 0u, 0u);
          id[k] = SINGLE ? src[k] : chunk_idx[src[k]];
          v[0][k] = a.x; v[1][k] = a.y; v[2][k] = a.z; v[3][k] = a.w;
          v[4][k] = b.x; v[5][k] = b.y; v[6][k] = b.z; v[7][k] = b.w;
        }
#pragma unroll
        for (int k = 0; k < kOver; ++k) {
          const uint32_t p = base + threadIdx.x + k * NT;
          uint32_t loc;
          if (pk) {
            loc = id[k] >> kIdxBits;
            id[k] = index_of(src[k], id[k]);
          } else {
            loc = cell_of(__uint_as_float(v[0][k]), __uint_as_float(v[1][k]), __uint_as_float(v[2][k]), g) - cell0;
          }
          if (!(p < count && loc < tc)) continue;
          if (SINGLE) keys_out[id[k]] = cell0 + loc;
          const size_t out = static_cast<size_t>(bs) + atomicAdd(&s_cnt[loc], 1u);
          if (out < n) {
            ordenado[out] = id[k];
            if (MOVE) {
              dst[out * 2u] = make_uint4(v[0][k], v[1][k], v[2][k], v[3][k]);
              dst[out * 2u + 1u] = make_uint4(v[4][k], v[5][k], v[6][k], v[7][k]);
            }
          }
        }
      }
    }
    if (STABLE && !shared) {
      // slots were taken in arrival order: every cell of two or more is
      // listed. Once every cursor is final it holds its cell's end, so a
      // cell's count is its end minus the previous cell's. The long cells
      // (tile-local numbers in s_idx, free now) then have their indices
      // copied to fl.idx() for the fix-up; a tile with more of them than
      // s_idx holds copies its whole range.
      if (threadIdx.x == 0) s_any_long = 0u;
      __syncthreads();
      list_cells_tile(2u, [&](uint32_t j) { return s_cnt[j] - (j ? s_cnt[j - 1u] : 0u); });
      for (uint32_t j = threadIdx.x; j < tc; j += NT) {
        const uint32_t len = s_cnt[j] - (j ? s_cnt[j - 1u] : 0u);
        if (len > kRankSortMax) {
          const uint32_t at = atomicAdd(&s_any_long, 1u);
          if (at < kStagedWin) s_idx[at] = j;
        }
      }
      __syncthreads();  // the list is whole, and this workgroup's ordenado stores are visible to it
      const uint32_t nl = s_any_long;
      const uint32_t places = n - bs;  // this tile's places that exist
      const uint32_t* from = ordenado + bs;
      uint32_t* to = fl.idx() + bs;
      for (uint32_t l = 0; l < ((nl <= kStagedWin) ? nl : 1u); ++l) {  // tile-uniform
        uint32_t a = 0u, e = count;
        if (nl <= kStagedWin) {
          const uint32_t j = s_idx[l];
          a = j ? s_cnt[j - 1u] : 0u;
          e = s_cnt[j];
        }
        e = (e < places) ? e : places;
        for (uint32_t q0 = a; q0 < e; q0 += NT * kStagedRegs) {
          uint32_t v[kStagedRegs];
#pragma unroll
          for (int k = 0; k < kStagedRegs; ++k) {
            const uint32_t loc = q0 + threadIdx.x + static_cast<uint32_t>(k) * NT;
            v[k] = (loc < e && loc >= q0) ? from[loc] : 0u;  // loc >= q0: no wrap past 2^32
          }
#pragma unroll
          for (int k = 0; k < kStagedRegs; ++k) {
            const uint32_t loc = q0 + threadIdx.x + static_cast<uint32_t>(k) * NT;
            if (loc < e && loc >= q0) to[loc] = v[k];
          }
        }
      }
    }
  }
}

}  // namespace ugp
