// kernels_reorder.h -- the gather reorder (gather mode, ugp_reorder and
// ugp_reorder_arrays) and the stable-order passes: the fix-up of the cells
// the tile kernel could not order itself (tile paths), and the per-cell
// sort after the atomic scatter (direct path).
#pragma once

#include "common.h"

namespace ugp {

constexpr int kGatherItems = 8;            // half-records per thread in the gather
constexpr uint32_t kSmallSort = 16;        // cells up to this length are sorted in registers
constexpr int kSortBlock = 1024;           // threads of the long-cell sort
constexpr uint32_t kLdsSort = 16384;       // longest cell sorted in LDS (64 KiB)
constexpr int kSortGrid = 512;             // workgroups of the long-cell sort (direct path)
constexpr uint32_t kRecBatch = 8;          // records gathered together by one thread (long cells)
constexpr uint32_t kBitmapPasses = 4;      // bitmap windows a long cell may take (2^21 index values)
constexpr uint32_t kMinPart = 1024;        // fewest places of a shared long cell one workgroup takes
constexpr uint32_t kOutStage = 8192;       // places of a long cell the fix-up orders in LDS before writing
// fix-up workgroups: 256 in all, one per CU (each takes ~97 KB of LDS), so
// that a fix-up with nothing listed is one round of workgroups that exit
constexpr uint32_t kFixLongBlocks = 32;    // on long cells (a cell of 10,000 takes 10)
constexpr uint32_t kFixShortBlocks = 224;  // on short cells

// Gather: two lanes per record, each moving one 16-byte half, so every
// store instruction writes a contiguous span, with the non-temporal hint
// (measured on MI355X: the gather of 1M records 24.9 -> 23.8 us). Indices
// >= n_src are skipped.
__global__ __launch_bounds__(kBlock) void gather_kernel(const uint32_t* __restrict__ idx, uint32_t n,
                                                        uint32_t n_src,
                                                        const uint4* __restrict__ src,
                                                        uint4* __restrict__ dst) {
  constexpr uint32_t kRecPerBlock = kBlock * kGatherItems / 2;
  const uint32_t base = blockIdx.x * kRecPerBlock;
  const uint32_t half = threadIdx.x & 1u;
  uint4 v[kGatherItems];
  uint32_t r[kGatherItems];
  bool ok[kGatherItems];
#pragma unroll
  for (int j = 0; j < kGatherItems; ++j) {
    r[j] = base + j * (kBlock / 2) + (threadIdx.x >> 1);
    const uint32_t s = idx[r[j] < n ? r[j] : n - 1u];
    ok[j] = (r[j] < n) && (s < n_src);
    v[j] = src[static_cast<size_t>(s < n_src ? s : n_src - 1u) * 2u + half];
  }
#pragma unroll
  for (int j = 0; j < kGatherItems; ++j)
    if (ok[j]) store_stream(dst + static_cast<size_t>(r[j]) * 2u + half, v[j]);
}

// Gather of several arrays with one index (page "Reordenar por celda y la
// coalescencia de memoria", section "El kernel de reordenación": a state
// split over several buffers is reordered in one kernel that reads each
// ordenado[k] once for all of them). Every element of every array is cut
// into chunks of sizeof(T) bytes (16 when every size and pointer allows,
// else 4); the W chunks of one destination element k, all arrays in turn,
// go to W consecutive threads, so a store instruction covers contiguous
// spans and ordenado[k] is read by those W threads together (one line).
// A workgroup handles kArrayItems groups of E = kBlock / W elements, the
// loads of all groups in flight before the first store. Indices >= n_src
// are skipped.
constexpr uint32_t kMaxArrays = 8;
constexpr int kArrayItems = 8;

struct ArraySet {
  const void* src[kMaxArrays];
  void* dst[kMaxArrays];
  uint32_t chunks[kMaxArrays];     // chunks per element of array q
  uint32_t first[kMaxArrays + 1];  // first[q]: chunk of array q within an element's W chunks
  uint32_t count;                  // arrays
};

template <typename T>
__global__ __launch_bounds__(kBlock) void gather_arrays_kernel(const uint32_t* __restrict__ idx,
                                                               uint32_t n, uint32_t n_src,
                                                               ArraySet a) {
  const uint32_t w_all = a.first[a.count];  // chunks per element, 1..kBlock
  const uint32_t per = kBlock / w_all;       // elements per group
  const uint32_t e = threadIdx.x / w_all, c = threadIdx.x - e * w_all;
  if (e >= per) return;  // no barrier below: idle lanes may leave
  uint32_t q = 0;
  while (q + 1 < a.count && a.first[q + 1] <= c) ++q;
  const uint32_t local = c - a.first[q], chunks = a.chunks[q];
  const T* src = static_cast<const T*>(a.src[q]);
  T* dst = static_cast<T*>(a.dst[q]);
  // register arrays as scalars (an array of 16-byte vectors is placed in
  // scratch memory by the compiler)
  uint32_t v0[kArrayItems], v1[kArrayItems], v2[kArrayItems], v3[kArrayItems];
  uint32_t k[kArrayItems];
  bool ok[kArrayItems];
#pragma unroll
  for (int j = 0; j < kArrayItems; ++j) {
    const uint64_t kk = (static_cast<uint64_t>(blockIdx.x) * kArrayItems + j) * per + e;
    k[j] = (kk < n) ? static_cast<uint32_t>(kk) : n - 1u;
    const uint32_t s = idx[k[j]];
    ok[j] = (kk < n) && (s < n_src);
    const T x = src[static_cast<size_t>(s < n_src ? s : n_src - 1u) * chunks + local];  // clamped, unconditional
    if constexpr (sizeof(T) == 16) {
      v0[j] = x.x; v1[j] = x.y; v2[j] = x.z; v3[j] = x.w;
    } else {
      v0[j] = x;
    }
  }
  // stores with the non-temporal hint (measured on MI355X: two 32-byte
  // arrays of 1M records 50.4 -> 49.4 us)
#pragma unroll
  for (int j = 0; j < kArrayItems; ++j) {
    if (!ok[j]) continue;
    T* d = dst + static_cast<size_t>(k[j]) * chunks + local;
    if constexpr (sizeof(T) == 16) {
      store_stream(d, make_uint4(v0[j], v1[j], v2[j], v3[j]));
    } else {
      store_stream(d, v0[j]);
    }
  }
}

// One thread puts a cell of 2..kSmallSort entries (slice [s, s + len) of
// ordenado) in index order: a bitonic network in registers on (particle
// index, position in the slice) pairs (static indices, padding with all
// ones, which no pair reaches). RECS: the records follow, read from `src`
// by position in the slice (BY_INDEX false: src holds the slice's records
// in its original order) or by particle index (BY_INDEX true: src is the
// input), BATCH records at a time.
template <bool RECS, bool BY_INDEX, uint32_t BATCH>
__device__ __forceinline__ void sort_cell_in_registers(uint32_t s, uint32_t len, uint32_t n,
                                                       uint32_t* __restrict__ ordenado,
                                                       const uint4* __restrict__ src,
                                                       uint4* __restrict__ reordered) {
  uint64_t v[kSmallSort];
#pragma unroll
  for (uint32_t k = 0; k < kSmallSort; ++k)
    v[k] = (k < len) ? (static_cast<uint64_t>(ordenado[s + k]) << 32) | k : ~0ull;
#pragma unroll
  for (uint32_t kk = 2; kk <= kSmallSort; kk <<= 1) {
#pragma unroll
    for (uint32_t j = kk >> 1; j > 0; j >>= 1) {
#pragma unroll
      for (uint32_t i = 0; i < kSmallSort; ++i) {
        const uint32_t l = i ^ j;
        if (l > i) {
          const bool up = (i & kk) == 0;
          const uint64_t a = v[i], b = v[l];
          if ((a > b) == up) {
            v[i] = b;
            v[l] = a;
          }
        }
      }
    }
  }
  // records BATCH at a time: a batch's loads are all in flight before
  // its stores (one wait per batch, not per record)
#pragma unroll
  for (uint32_t k0 = 0; k0 < kSmallSort; k0 += BATCH) {
    uint4 ra[BATCH], rb[BATCH];
#pragma unroll
    for (uint32_t j = 0; j < BATCH; ++j) ra[j] = rb[j] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (uint32_t j = 0; j < BATCH; ++j) {
      const uint32_t k = k0 + j, idx = static_cast<uint32_t>(v[k] >> 32);
      if (RECS && k < len && (!BY_INDEX || idx < n)) {
        const size_t from = BY_INDEX ? 2ull * idx : 2ull * (s + static_cast<uint32_t>(v[k] & 0xFFFFFFFFu));
        ra[j] = src[from];
        rb[j] = src[from + 1u];
      }
    }
#pragma unroll
    for (uint32_t j = 0; j < BATCH; ++j) {
      const uint32_t k = k0 + j, idx = static_cast<uint32_t>(v[k] >> 32);
      if (k < len) {
        ordenado[s + k] = idx;
        if (RECS && (!BY_INDEX || idx < n)) {
          reordered[2ull * (s + k)] = ra[j];
          reordered[2ull * (s + k) + 1u] = rb[j];
        }
      }
    }
  }
}

// Stable mode, short cells: one thread per cell. Cells of at most 16
// entries are sorted in registers (sort_cell_in_registers); longer cells
// are appended to a list for the LDS kernel. RECS: the scatter kernel left the records in `unstable` in the
// slice's original order, and each short cell writes its records to
// `reordered` in the sorted order (reads stay inside the cell's slice);
// the long-cell kernel writes the records of long cells.
template <bool RECS>
__global__ __launch_bounds__(kBlock) void sort_short_cells_kernel(
    const uint32_t* __restrict__ inicios, uint32_t cells, uint32_t n,
    uint32_t* __restrict__ ordenado, uint32_t* __restrict__ long_list, uint32_t long_cap,
    uint32_t* __restrict__ long_count, const uint4* __restrict__ unstable, uint4* __restrict__ reordered) {
  const uint32_t c = blockIdx.x * kBlock + threadIdx.x;
  if (c >= cells) return;
  const uint32_t s = inicios[c];
  const uint32_t e = inicios[c + 1];
  if (e > n || e <= s) return;
  const uint32_t len = e - s;
  if (len > kSmallSort) {
    const uint32_t k = atomicAdd(long_count, 1u);
    if (k < long_cap) long_list[k] = c;
    return;
  }
  if (len == 1) {
    if (RECS) {
      reordered[2ull * s] = unstable[2ull * s];
      reordered[2ull * s + 1u] = unstable[2ull * s + 1u];
    }
    return;
  }
  sort_cell_in_registers<RECS, false, 4>(s, len, n, ordenado, unstable, reordered);
}

// The records of a long cell once its indices are in order: the workgroup
// reads ordenado[s, s + len) back (its own writes, visible after the
// barrier) and gathers kRecBatch records per thread at a time. Ends with a
// barrier.
__device__ __forceinline__ void copy_cell_records(uint32_t s, uint32_t len, uint32_t n,
                                                  const uint32_t* __restrict__ ordenado,
                                                  const uint4* __restrict__ particles,
                                                  uint4* __restrict__ reordered) {
  __syncthreads();
  for (uint32_t t0 = threadIdx.x; t0 < len; t0 += kRecBatch * kSortBlock) {
    uint32_t id[kRecBatch];
    uint4 ra[kRecBatch], rb[kRecBatch];
#pragma unroll
    for (uint32_t j = 0; j < kRecBatch; ++j) {
      const uint32_t t = t0 + j * kSortBlock;
      id[j] = (t < len) ? ordenado[s + t] : 0xFFFFFFFFu;
      ra[j] = rb[j] = make_uint4(0u, 0u, 0u, 0u);
      if (id[j] < n) {
        ra[j] = particles[2ull * id[j]];
        rb[j] = particles[2ull * id[j] + 1u];
      }
    }
#pragma unroll
    for (uint32_t j = 0; j < kRecBatch; ++j) {
      const uint32_t t = t0 + j * kSortBlock;
      if (t < len && id[j] < n) {
        reordered[2ull * (s + t)] = ra[j];
        reordered[2ull * (s + t) + 1u] = rb[j];
      }
    }
  }
  __syncthreads();
}

// The places [s, s + len) of a long cell whose indices, in order, are in
// LDS (ids): ordenado and the records gathered from the input by index are
// written contiguously, kRecBatch records per thread at a time. Ends with
// a barrier.
__device__ __forceinline__ void write_cell_from_lds(uint32_t s, uint32_t len, uint32_t n, const uint32_t* ids,
                                                    uint32_t* __restrict__ ordenado,
                                                    const uint4* __restrict__ particles,
                                                    uint4* __restrict__ reordered, bool recs) {
  for (uint32_t t0 = threadIdx.x; t0 < len; t0 += kRecBatch * kSortBlock) {
    uint32_t id[kRecBatch];
    uint4 ra[kRecBatch], rb[kRecBatch];
#pragma unroll
    for (uint32_t j = 0; j < kRecBatch; ++j) {
      const uint32_t t = t0 + j * kSortBlock;
      id[j] = (t < len) ? ids[t] : 0xFFFFFFFFu;
      if (t < len) ordenado[s + t] = id[j];
      ra[j] = rb[j] = make_uint4(0u, 0u, 0u, 0u);
      if (recs && id[j] < n) {
        ra[j] = particles[2ull * id[j]];
        rb[j] = particles[2ull * id[j] + 1u];
      }
    }
    if (recs) {
#pragma unroll
      for (uint32_t j = 0; j < kRecBatch; ++j) {
        const uint32_t t = t0 + j * kSortBlock;
        if (t < len && id[j] < n) {
          reordered[2ull * (s + t)] = ra[j];
          reordered[2ull * (s + t) + 1u] = rb[j];
        }
      }
    }
  }
  __syncthreads();
}

// Stable mode, long cells: the workgroups first, first + stride, ... take
// entries first, first + stride, ... of the list of long cells. Up to 16384
// entries, held in registers: when the cell's indices span at most
// kBitmapPasses * 2^19 values, a bitmap of one such window at a time in LDS
// (s_keys): each index sets its bit, wave scans of the words' set bits and
// a scan of the wave totals (s_tab) give each word the number of set bits
// before it (s_pre, 16 bits per word), and each index's place is that
// number plus the set bits below it in its own word, so every thread places
// its own indices with no serial walk over the bits (a dense cell would put
// hundreds of bits in one thread's words). Otherwise a bitonic sort in LDS.
// Longer: ordered compaction, i.e. walk all particles in index order and
// append those of this cell (the cell's membership is exact already; only
// order changes). Each way writes indices only; RECS: the records follow in
// one pass over the ordered slice (copy_cell_records). With the bitmap and
// s_out (kOutStage words of LDS, or nullptr), a part of up to kOutStage
// places is ordered in LDS first and written out contiguously, records
// gathered by the indices held there (write_cell_from_lds).
//
// SHARE: the cell's arrival-order indices are read from `arrival` (at the
// same places), which nothing writes meanwhile, so with fewer cells than
// workgroups stride / count workgroups can share a cell of up to kLdsSort
// (at least kMinPart entries each): with the bitmap, each takes an equal
// part of the cell's index range, counts the cell's indices below it (its
// first place) and in it, and orders only those; with the bitonic sort,
// each sorts the whole cell and keeps an equal share of the places. Each
// writes and gathers only its own places. No workgroup waits for another.
// Without SHARE the indices are read from ordenado itself and a cell has
// one workgroup.
template <bool RECS, bool SHARE>
__device__ __forceinline__ void sort_long_cells(
    const uint32_t* __restrict__ inicios, const uint32_t* __restrict__ celdaDe, uint32_t n,
    const uint32_t* __restrict__ long_list, uint32_t count, uint32_t first, uint32_t stride,
    const uint32_t* arrival, uint32_t* __restrict__ ordenado, const uint4* __restrict__ particles,
    uint4* __restrict__ reordered, uint32_t* s_keys, uint16_t* s_pre, uint32_t* s_tab, uint32_t* s_wave,
    uint32_t* s_out) {
  const uint32_t* src = SHARE ? arrival : ordenado;
  uint32_t share = 1, part = 0;
  if (SHARE && count != 0u && count < stride) {
    share = stride / count;
    part = first % share;
    first /= share;
    stride = count;  // one cell per workgroup
  }
  for (uint32_t k = first; k < count; k += stride) {
    const uint32_t c = long_list[k];
    const uint32_t s = inicios[c];
    const uint32_t e = inicios[c + 1];
    if (e <= s || e > n) continue;  // uniform across the workgroup
    const uint32_t len = e - s;
    uint32_t parts = 1;
    if (len <= kLdsSort) {
      parts = (len + kMinPart - 1u) / kMinPart;
      parts = (parts < share) ? parts : share;
    }
    if (part >= parts) continue;
    const uint32_t p0 = static_cast<uint32_t>(static_cast<uint64_t>(len) * part / parts);
    const uint32_t p1 = static_cast<uint32_t>(static_cast<uint64_t>(len) * (part + 1u) / parts);
    if (len <= kLdsSort) {
      constexpr uint32_t kPer = kLdsSort / kSortBlock;  // entries (and bitmap words) per thread
      constexpr uint32_t kWindow = kLdsSort * 32u;      // indices per bitmap window
      constexpr uint32_t kWaves = kSortBlock / 64;
      const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
      uint32_t v[kPer];
      uint32_t lo = 0xFFFFFFFFu, hi = 0;
#pragma unroll
      for (uint32_t q = 0; q < kPer; ++q) {
        const uint32_t t = threadIdx.x + q * kSortBlock;
        v[q] = (t < len) ? src[s + t] : 0u;
        if (t < len) {
          lo = (v[q] < lo) ? v[q] : lo;
          hi = (v[q] > hi) ? v[q] : hi;
        }
      }
      lo = ~block_max<kSortBlock>(~lo, s_wave);
      hi = block_max<kSortBlock>(hi, s_wave);
      if (hi - lo < kBitmapPasses * kWindow) {  // len >= 1, so lo <= hi; uniform
        // this workgroup's part [w_lo, w_end) of the index range (the whole
        // range unshared; empty only if the cell repeats an index) and its
        // places [q0, q1): the cell's indices below w_lo come first
        const uint64_t span = static_cast<uint64_t>(hi - lo) + 1u;
        const uint64_t w_lo = lo + span * part / parts;
        const uint64_t w_end = lo + span * (part + 1u) / parts;  // <= hi + 1 <= 2^32
        uint32_t below = 0, inside = 0;
#pragma unroll
        for (uint32_t q = 0; q < kPer; ++q) {
          if (threadIdx.x + q * kSortBlock < len) {
            below += (v[q] < w_lo) ? 1u : 0u;
            inside += (v[q] >= w_lo && v[q] < w_end) ? 1u : 0u;
          }
        }
        const uint32_t packed = block_sum<kSortBlock>(below | (inside << 16), s_wave);  // each <= kLdsSort < 2^16
        const uint32_t q0 = packed & 0xFFFFu, q1 = q0 + (packed >> 16);
        const bool staged = s_out != nullptr && q1 - q0 <= kOutStage;  // uniform
        uint32_t placed = q0;
        for (uint64_t base64 = w_lo; base64 < w_end; base64 += kWindow) {
          const uint32_t base = static_cast<uint32_t>(base64);  // < w_end <= 2^32: fits
          // the bitmap words this window's part of the range can touch;
          // thread t owns words t, t + kSortBlock, ... (a wave's lanes touch
          // consecutive words: no LDS bank conflicts)
          const uint64_t last = w_end - 1u - base64;
          const uint32_t top = (last < kWindow - 1u) ? static_cast<uint32_t>(last) : kWindow - 1u;
          const uint32_t used = (top >> 5) + 1u;
          const uint32_t nq = (used + kSortBlock - 1u) / kSortBlock;  // word groups in use (<= kPer)
          for (uint32_t q = 0; q < nq; ++q)
            if (q * kSortBlock + threadIdx.x < used) s_keys[q * kSortBlock + threadIdx.x] = 0u;
          __syncthreads();
#pragma unroll 4
          for (uint32_t q = 0; q < kPer; ++q) {
            const uint32_t off = v[q] - base;  // wraps (and fails the test) below the window
            if (threadIdx.x + q * kSortBlock < len && v[q] >= base && off <= top)
              atomicOr(&s_keys[off >> 5], 1u << (off & 31u));
          }
          __syncthreads();
          // s_pre[word] = set bits in the words before it. Words in order
          // are groups q of kSortBlock, each the 64-word runs of the waves:
          // a wave scan places a word inside its run, and an exclusive scan
          // of the run totals in (q, wave) order (s_tab) places the runs.
          for (uint32_t q = 0; q < nq; ++q) {
            const uint32_t wd = q * kSortBlock + threadIdx.x;
            const uint32_t incl = wave_inclusive_sum((wd < used) ? __popc(s_keys[wd]) : 0u);
            if (lane == 63u) s_tab[q * kWaves + wave] = incl;
          }
          __syncthreads();
          uint32_t total;
          {
            const uint32_t x = (threadIdx.x < nq * kWaves) ? s_tab[threadIdx.x] : 0u;
            const uint32_t ex = block_exclusive_sum<kSortBlock>(x, s_wave, &total);
            if (threadIdx.x < nq * kWaves) s_tab[threadIdx.x] = ex;  // its own entry only
          }
          __syncthreads();
          for (uint32_t q = 0; q < nq; ++q) {
            const uint32_t wd = q * kSortBlock + threadIdx.x;
            const uint32_t c = (wd < used) ? __popc(s_keys[wd]) : 0u;
            const uint32_t incl = wave_inclusive_sum(c);
            if (wd < used) s_pre[wd] = static_cast<uint16_t>(s_tab[q * kWaves + wave] + incl - c);  // < kLdsSort
          }
          __syncthreads();
          // every index's place: the indices below its word plus the set
          // bits below it in its word
#pragma unroll 4
          for (uint32_t q = 0; q < kPer; ++q) {
            const uint32_t off = v[q] - base;
            if (threadIdx.x + q * kSortBlock < len && v[q] >= base && off <= top) {
              const uint32_t wd = off >> 5;
              const uint32_t place =
                  placed + s_pre[wd] + __popc(s_keys[wd] & ((1u << (off & 31u)) - 1u));
              if (place < q1) {  // < len: distinct indices
                if (staged)
                  s_out[place - q0] = v[q];
                else
                  ordenado[s + place] = v[q];
              }
            }
          }
          placed += total;
          __syncthreads();  // this window's reads end before the next one is cleared
        }
        if (staged)
          write_cell_from_lds(s + q0, q1 - q0, n, s_out, ordenado, particles, reordered, RECS);
        else if (RECS)
          copy_cell_records(s + q0, q1 - q0, n, ordenado, particles, reordered);
        continue;
      }
      uint32_t L = 1;
      while (L < len) L <<= 1;
      for (uint32_t t = threadIdx.x; t < L; t += kSortBlock)
        s_keys[t] = (t < len) ? src[s + t] : 0xFFFFFFFFu;
      __syncthreads();
      for (uint32_t kk = 2; kk <= L; kk <<= 1) {
        for (uint32_t j = kk >> 1; j > 0; j >>= 1) {
          for (uint32_t t = threadIdx.x; t < (L >> 1); t += kSortBlock) {
            const uint32_t i = ((t & ~(j - 1u)) << 1) | (t & (j - 1u));  // j is a power of two
            const uint32_t l = i + j;
            const bool up = (i & kk) == 0;
            const uint32_t a = s_keys[i], b = s_keys[l];
            if ((a > b) == up) {
              s_keys[i] = b;
              s_keys[l] = a;
            }
          }
          __syncthreads();
        }
      }
      for (uint32_t t = p0 + threadIdx.x; t < p1; t += kSortBlock) ordenado[s + t] = s_keys[t];
      if (RECS) copy_cell_records(s + p0, p1 - p0, n, ordenado, particles, reordered);
      __syncthreads();
    } else {
      uint32_t run = 0;
      for (uint64_t b0 = 0; b0 < n; b0 += kSortBlock) {
        const uint64_t i = b0 + threadIdx.x;
        const uint32_t flag = (i < n && celdaDe[i] == c) ? 1u : 0u;
        uint32_t total;
        const uint32_t excl = block_exclusive_sum<kSortBlock>(flag, s_wave, &total);
        const uint32_t dst = s + run + excl;
        if (flag && dst < e) ordenado[dst] = static_cast<uint32_t>(i);
        run += total;
      }
      if (RECS) copy_cell_records(s, len, n, ordenado, particles, reordered);
    }
  }
}

// The long-cell pass of the direct path: one workgroup per listed cell.
template <bool RECS>
__global__ __launch_bounds__(kSortBlock) void sort_long_cells_kernel(
    const uint32_t* __restrict__ inicios, const uint32_t* __restrict__ celdaDe, uint32_t n,
    const uint32_t* __restrict__ long_list, uint32_t long_cap,
    const uint32_t* __restrict__ long_count, uint32_t* __restrict__ ordenado,
    const uint4* __restrict__ particles, uint4* __restrict__ reordered) {
  __shared__ uint32_t s_keys[kLdsSort];
  __shared__ uint16_t s_pre[kLdsSort];
  __shared__ uint32_t s_tab[kLdsSort / 64];
  __shared__ uint32_t s_wave[kSortBlock / 64];
  uint32_t count = *long_count;
  if (count > long_cap) count = long_cap;
  sort_long_cells<RECS, false>(inicios, celdaDe, n, long_list, count, blockIdx.x, gridDim.x, nullptr, ordenado,
                               particles, reordered, s_keys, s_pre, s_tab, s_wave, nullptr);
}

// Stable mode on the tile paths: the one pass over the cells the tile
// kernel left in arrival order (FixLists). Workgroups below long_blocks
// take the long cells (sort_long_cells, reading the arrival order from
// fl.idx(), so that several of them can share one cell). In the others the
// listed short cells are permuted in place inside their slices, where the
// tile kernel put their indices and (RECS) records: groups of 16 lanes take
// the cells of up to kSmallSort (lane j holds entry j; its place is the
// number of smaller indices among the group's, counted with lane shuffles),
// then whole waves take the cells of up to kRankSortMax (each lane holds up
// to kRankSortMax / 64 entries; the cell's indices go to the wave's LDS
// slice and each lane counts the ones below its own). Every entry is read
// before any is written back, so the permutation in place is safe. LDS is
// shared by the two roles.
template <bool RECS>
__global__ __launch_bounds__(kSortBlock) void fix_cells_kernel(
    const uint32_t* __restrict__ inicios, const uint32_t* __restrict__ celdaDe, uint32_t cells, uint32_t n,
    FixLists fl, uint32_t long_blocks, uint32_t* __restrict__ ordenado, const uint4* __restrict__ particles,
    uint4* __restrict__ reordered) {
  constexpr uint32_t kWaves = kSortBlock / 64;
  static_assert(kWaves * kRankSortMax <= kLdsSort, "one slice per wave fits the long-cell buffer");
  constexpr uint32_t kWaveEntries = kRankSortMax / 64;  // entries per lane in the wave pass
  static_assert(kRankSortMax % 64 == 0, "whole entries per lane");
  static_assert(kSmallSort == 16, "one group of 16 lanes per short cell");
  __shared__ __align__(16) uint32_t s_keys[kLdsSort];  // slices read as uint4
  __shared__ uint16_t s_pre[kLdsSort];
  __shared__ uint32_t s_tab[kLdsSort / 64];
  __shared__ uint32_t s_wave[kWaves];
  __shared__ uint32_t s_out[kOutStage];  // a long cell's ordered places before they are written
  if (blockIdx.x < long_blocks) {
    uint32_t count = fl.counts()[1];
    if (count > fl.long_cap) count = fl.long_cap;
    sort_long_cells<RECS, true>(inicios, celdaDe, n, fl.lng(), count, blockIdx.x, long_blocks, fl.idx(),
                                ordenado, particles, reordered, s_keys, s_pre, s_tab, s_wave, s_out);
    return;
  }
  const uint32_t lane = threadIdx.x & 63u;
  uint32_t* slice = s_keys + (threadIdx.x >> 6) * kRankSortMax;
  uint32_t count = fl.counts()[0];
  if (count > fl.fix_cap) count = fl.fix_cap;
  // cell of list entry k: {start, length} when it is one this role takes
  auto listed = [&](uint32_t k) -> uint2 {
    const uint32_t c = fl.fix()[k];
    if (c >= cells) return make_uint2(0u, 0u);
    const uint32_t a = inicios[c], e = inicios[c + 1];
    return (e > a && e <= n && e - a <= kRankSortMax) ? make_uint2(a, e - a) : make_uint2(0u, 0u);
  };
  // The role's workgroups take the list entries in turn (entry k to
  // workgroup k mod role_wgs), a batch of kSortBlock of them at a time: every
  // thread reads one entry's slice into an LDS table (one round of loads for
  // the whole batch), the longer cells are gathered into a second table, and
  // then the groups take the short cells and the waves, one at a time from
  // an LDS counter, the longer ones, so that a wave's work follows the cells'
  // sizes rather than the order of the list.
  const uint32_t role_wg = blockIdx.x - long_blocks, role_wgs = gridDim.x - long_blocks;
  uint2* s_cells = reinterpret_cast<uint2*>(s_keys + kWaves * kRankSortMax);  // kSortBlock slices
  uint32_t* s_med = s_keys + kWaves * kRankSortMax + 2u * kSortBlock;         // the batch's longer cells
  static_assert(kWaves * kRankSortMax + 3u * kSortBlock <= kLdsSort, "the batch tables fit beside the slices");
  const uint32_t gl = threadIdx.x & 15u;
  for (uint64_t b0 = 0; role_wg + b0 * role_wgs < count; b0 += kSortBlock) {  // uniform
    __syncthreads();  // the previous batch's tables are read
    if (threadIdx.x == 0) {
      s_tab[0] = 0u;  // longer cells in the batch
      s_tab[1] = 0u;  // the next of them to take
    }
    __syncthreads();
    const uint64_t kk = role_wg + (b0 + threadIdx.x) * role_wgs;
    const uint2 mine_cell = (kk < count) ? listed(static_cast<uint32_t>(kk)) : make_uint2(0u, 0u);
    s_cells[threadIdx.x] = mine_cell;
    if (mine_cell.y > kSmallSort) s_med[atomicAdd(&s_tab[0], 1u)] = threadIdx.x;
    __syncthreads();
    // groups of 16 lanes: the batch's cells of up to kSmallSort
    for (uint32_t ci = threadIdx.x >> 4; ci < kSortBlock; ci += kSortBlock / 16u) {  // uniform across the group
      const uint2 sl = s_cells[ci];
      if (sl.y < 2u || sl.y > kSmallSort) continue;
      const bool has = gl < sl.y;
      const uint32_t mine = has ? ordenado[sl.x + gl] : 0xFFFFFFFFu;  // all ones: no index reaches it
      uint4 ra = make_uint4(0u, 0u, 0u, 0u), rb = ra;
      if (RECS && has) {
        ra = reordered[2ull * (sl.x + gl)];
        rb = reordered[2ull * (sl.x + gl) + 1u];
      }
      __builtin_amdgcn_s_waitcnt(kWaitLoadsAndStores);  // every entry read before any is written back
      uint32_t rank = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) rank += (static_cast<uint32_t>(__shfl(static_cast<int>(mine), i, 16)) < mine) ? 1u : 0u;
      if (has) {
        ordenado[sl.x + rank] = mine;
        if (RECS) {
          reordered[2ull * (sl.x + rank)] = ra;
          reordered[2ull * (sl.x + rank) + 1u] = rb;
        }
      }
    }
    // whole waves: the batch's cells of kSmallSort + 1 .. kRankSortMax
    const uint32_t nmed = s_tab[0];
    for (;;) {  // uniform across the wave
      uint32_t j = 0;
      if (lane == 0u) j = atomicAdd(&s_tab[1], 1u);
      j = static_cast<uint32_t>(__shfl(static_cast<int>(j), 0));
      if (j >= nmed) break;
      const uint2 sl = s_cells[s_med[j]];
      const uint32_t cs = sl.x, cl = sl.y, cl4 = (cl + 3u) & ~3u;
      uint32_t mine[kWaveEntries];
      uint4 ra[kWaveEntries], rb[kWaveEntries];
#pragma unroll
      for (uint32_t g = 0; g < kWaveEntries; ++g) {
        const uint32_t q = g * 64u + lane;
        mine[g] = (q < cl) ? ordenado[cs + q] : 0xFFFFFFFFu;  // all ones pads the slice: no index reaches it
        ra[g] = rb[g] = make_uint4(0u, 0u, 0u, 0u);
        if (RECS && q < cl) {
          ra[g] = reordered[2ull * (cs + q)];
          rb[g] = reordered[2ull * (cs + q) + 1u];
        }
      }
      __builtin_amdgcn_s_waitcnt(kWaitLoadsAndStores);  // every entry read before any is written back
#pragma unroll
      for (uint32_t g = 0; g < kWaveEntries; ++g)
        if (g * 64u + lane < cl4) slice[g * 64u + lane] = mine[g];
      // a wave's LDS accesses complete in order: the slice is whole for
      // every lane after this point
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (uint32_t g = 0; g < kWaveEntries; ++g) {
        const uint32_t q = g * 64u + lane;
        if (g * 64u < cl) {  // uniform across the wave
          uint32_t rank = 0;
          for (uint32_t j = 0; j < cl4; j += 4u) {  // the same address for every lane
            const uint4 w4 = *reinterpret_cast<const uint4*>(slice + j);
            rank += (w4.x < mine[g] ? 1u : 0u) + (w4.y < mine[g] ? 1u : 0u) + (w4.z < mine[g] ? 1u : 0u) +
                    (w4.w < mine[g] ? 1u : 0u);
          }
          if (q < cl) {
            ordenado[cs + rank] = mine[g];
            if (RECS) {
              reordered[2ull * (cs + rank)] = ra[g];
              reordered[2ull * (cs + rank) + 1u] = rb[g];
            }
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();  // every read of the slice before the next cell's writes
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

}  // namespace ugp
