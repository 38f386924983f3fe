// kernels_reorder.h -- the gather reorder and the stable-order pass.
#pragma once

#include "common.h"

namespace ugp {

constexpr int kGatherItems = 8;      // half-records per thread in the gather
constexpr uint32_t kSmallSort = 16;  // cells up to this length are sorted in registers
constexpr int kSortBlock = 1024;     // threads of the long-cell sort
constexpr uint32_t kLdsSort = 16384; // longest cell sorted in LDS (64 KiB)
constexpr int kSortGrid = 512;       // workgroups of the long-cell sort

// Gather: two lanes per record, each moving one 16-byte half, so every
// store instruction writes a contiguous span. Indices >= n_src are skipped.
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
    if (ok[j]) dst[static_cast<size_t>(r[j]) * 2u + half] = v[j];
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
#pragma unroll
  for (int j = 0; j < kArrayItems; ++j) {
    if (!ok[j]) continue;
    T* d = dst + static_cast<size_t>(k[j]) * chunks + local;
    if constexpr (sizeof(T) == 16) {
      *d = make_uint4(v0[j], v1[j], v2[j], v3[j]);
    } else {
      *d = v0[j];
    }
  }
}

// Stable mode, short cells: one thread per cell. Cells of at most 16
// entries are sorted in registers with a bitonic network on (particle
// index, position in the slice) pairs (static indices, padding with all
// ones, which no pair reaches); longer cells are appended to a list for the
// LDS kernel. RECS: the scatter kernel left the records in `unstable` in the
// slice's original order, and each short cell writes its records to
// `reordered` in the sorted order (reads stay inside the cell's slice);
// the long-cell kernel writes the records of long cells.
//
// LISTED: only the cells of `listed` (its first min(*listed_count,
// listed_cap) entries; the tile kernel appended the cells it could not sort
// itself), and their
// records come from the input particles by index (`unstable` then points to
// the particles) instead of from a copy by position.
template <bool RECS, bool LISTED>
__global__ __launch_bounds__(kBlock) void sort_short_cells_kernel(
    const uint32_t* __restrict__ inicios, uint32_t cells, uint32_t n,
    uint32_t* __restrict__ ordenado, uint32_t* __restrict__ long_list, uint32_t long_cap,
    uint32_t* __restrict__ long_count, const uint4* __restrict__ unstable, uint4* __restrict__ reordered,
    const uint32_t* __restrict__ listed, const uint32_t* __restrict__ listed_count,
    uint32_t listed_cap) {
  const uint32_t tid = blockIdx.x * kBlock + threadIdx.x;
  if (LISTED && (tid >= *listed_count || tid >= listed_cap)) return;
  const uint32_t c = LISTED ? listed[tid] : tid;
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
    if (RECS && !LISTED) {
      reordered[2ull * s] = unstable[2ull * s];
      reordered[2ull * s + 1u] = unstable[2ull * s + 1u];
    }
    return;
  }
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
#pragma unroll
  for (uint32_t k = 0; k < kSmallSort; ++k) {
    if (k < len) {
      ordenado[s + k] = static_cast<uint32_t>(v[k] >> 32);
      if (RECS) {
        const size_t from = LISTED ? 2ull * static_cast<uint32_t>(v[k] >> 32)
                                   : 2ull * (s + static_cast<uint32_t>(v[k] & 0xFFFFFFFFu));
        const uint4 a = unstable[from], b = unstable[from + 1u];
        reordered[2ull * (s + k)] = a;
        reordered[2ull * (s + k) + 1u] = b;
      }
    }
  }
}

// Stable mode, long cells: one workgroup per listed cell (grid-stride over
// the list). Up to 16384 entries: bitonic sort in LDS. Longer: ordered
// compaction, i.e. walk all particles in index order and append those of
// this cell (the cell's membership is exact already; only order changes).
// RECS: each sorted entry's record is copied from the input particles.
template <bool RECS>
__global__ __launch_bounds__(kSortBlock) void sort_long_cells_kernel(
    const uint32_t* __restrict__ inicios, const uint32_t* __restrict__ celdaDe, uint32_t n,
    const uint32_t* __restrict__ long_list, uint32_t long_cap,
    const uint32_t* __restrict__ long_count, uint32_t* __restrict__ ordenado,
    const uint4* __restrict__ particles, uint4* __restrict__ reordered) {
  __shared__ uint32_t s_keys[kLdsSort];
  __shared__ uint32_t s_wave[kSortBlock / 64];
  uint32_t count = *long_count;
  if (count > long_cap) count = long_cap;
  for (uint32_t k = blockIdx.x; k < count; k += gridDim.x) {
    const uint32_t c = long_list[k];
    const uint32_t s = inicios[c];
    const uint32_t e = inicios[c + 1];
    if (e <= s || e > n) continue;  // uniform across the workgroup
    const uint32_t len = e - s;
    if (len <= kLdsSort) {
      uint32_t L = 1;
      while (L < len) L <<= 1;
      for (uint32_t t = threadIdx.x; t < L; t += kSortBlock)
        s_keys[t] = (t < len) ? ordenado[s + t] : 0xFFFFFFFFu;
      __syncthreads();
      for (uint32_t kk = 2; kk <= L; kk <<= 1) {
        for (uint32_t j = kk >> 1; j > 0; j >>= 1) {
          for (uint32_t t = threadIdx.x; t < (L >> 1); t += kSortBlock) {
            const uint32_t i = (t / j) * (2 * j) + (t % j);
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
      for (uint32_t t = threadIdx.x; t < len; t += kSortBlock) {
        const uint32_t idx = s_keys[t];
        ordenado[s + t] = idx;
        if (RECS && idx < n) {
          reordered[2ull * (s + t)] = particles[2ull * idx];
          reordered[2ull * (s + t) + 1u] = particles[2ull * idx + 1u];
        }
      }
      __syncthreads();
    } else {
      uint32_t run = 0;
      for (uint64_t b0 = 0; b0 < n; b0 += kSortBlock) {
        const uint64_t i = b0 + threadIdx.x;
        const uint32_t flag = (i < n && celdaDe[i] == c) ? 1u : 0u;
        uint32_t total;
        const uint32_t excl = block_exclusive_sum<kSortBlock>(flag, s_wave, &total);
        const uint32_t dst = s + run + excl;
        if (flag && dst < e) {
          ordenado[dst] = static_cast<uint32_t>(i);
          if (RECS) {
            reordered[2ull * dst] = particles[2u * i];
            reordered[2ull * dst + 1u] = particles[2u * i + 1u];
          }
        }
        run += total;
      }
    }
  }
}

}  // namespace ugp
