// kernels_diag.h -- overflow diagnostics of a finished histogram (page
// "Contar partículas por celda", section "Detectar el desbordamiento sin
// salir de la GPU").
//
// Two numbers: the largest occupancy of any cell, and how many insertions
// found their cell already holding `capacity` particles or more. Inserting
// the k-th particle of a cell leaves it with occupancy k and overflows when
// k > capacity, so a cell of m particles contributes max(0, m - capacity)
// overflows in any insertion order, and the largest occupancy is the largest
// count. Both are therefore reductions over conteos: this file holds the
// wave reductions, the per-workgroup publication (one atomic max and at most
// one atomic add per workgroup into two words zeroed beforehand), and a
// standalone kernel over a conteos array. The staged tile kernel applies the
// same reduction to its LDS histogram instead (no extra traffic).
#pragma once

#include "common.h"

namespace ugp {

__device__ __forceinline__ uint32_t overflow_of(uint32_t count, uint32_t cap) {
  return count > cap ? count - cap : 0u;
}

// Reductions across the 64 lanes of a wave (every lane gets the result).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t y = static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), o, 64));
    x = (y > x) ? y : x;
  }
  return x;
}
__device__ __forceinline__ uint32_t wave_add_u32(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), o, 64));
  return x;
}

// Thread 0 of a workgroup folds the per-wave partials (s_m, s_o: one word per
// wave, written before the last barrier) and publishes them.
template <int NT>
__device__ __forceinline__ void publish_diag(const uint32_t* s_m, const uint32_t* s_o,
                                             uint32_t* diag) {
  if (threadIdx.x != 0) return;
  uint32_t m = 0, o = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    m = (s_m[w] > m) ? s_m[w] : m;
    o += s_o[w];
  }
  atomicMax(&diag[0], m);
  if (o != 0u) atomicAdd(&diag[1], o);
}

// Standalone reduction over a conteos array in one launch, with no clear
// beforehand: every workgroup folds its part and stores the pair in its
// entry of `part`, then takes a ticket; the workgroup that takes the last
// ticket folds the gridDim.x pairs, writes diag[0] (largest count) and
// diag[1] (sum of max(0, count - cap)) and puts the ticket back to zero for
// the next launch. ticket/part: one slot of a library-owned device array
// (zero at load, zero again after every launch); at most kDiagGrid
// workgroups. conteos 16-byte aligned. Each thread issues kDiagItems
// 16-byte loads per round before using any of them.
constexpr int kDiagItems = 4;
constexpr int kDiagThreads = 512;
constexpr uint32_t kDiagGrid = 256;  // workgroups at most (one partial each)
constexpr uint32_t kDiagRounds = 2;  // load rounds per workgroup below that cap
constexpr uint32_t kDiagSlots = 64;  // launches that may be in flight at once on one GPU
struct DiagScratch {
  uint32_t ticket[kDiagSlots];
  uint2 part[kDiagSlots][kDiagGrid];
};

template <int NT>
__global__ __launch_bounds__(NT) void cell_diag_kernel(const uint32_t* __restrict__ conteos, uint32_t cells,
                                                       uint32_t cap, uint32_t* __restrict__ diag,
                                                       uint32_t* ticket, uint2* part) {
  static_assert(kDiagGrid <= static_cast<uint32_t>(NT), "the last workgroup folds one partial per thread");
  __shared__ uint32_t s_m[NT / 64], s_o[NT / 64];
  __shared__ uint32_t s_last;
  uint32_t m = 0, o = 0;
  const uint64_t nvec = cells / 4u;
  const uint64_t round = static_cast<uint64_t>(gridDim.x) * NT * kDiagItems;
  const uint4* c4 = reinterpret_cast<const uint4*>(conteos);
  for (uint64_t q0 = static_cast<uint64_t>(blockIdx.x) * NT * kDiagItems + threadIdx.x; q0 < nvec;
       q0 += round) {
    uint4 v[kDiagItems];
#pragma unroll
    for (int k = 0; k < kDiagItems; ++k) {
      const uint64_t q = q0 + static_cast<uint64_t>(k) * NT;
      v[k] = (q < nvec) ? load_stream(c4 + q) : make_uint4(0u, 0u, 0u, 0u);  // 0 adds nothing
    }
#pragma unroll
    for (int k = 0; k < kDiagItems; ++k) {
      const uint32_t a = (v[k].x > v[k].y) ? v[k].x : v[k].y;
      const uint32_t b = (v[k].z > v[k].w) ? v[k].z : v[k].w;
      const uint32_t ab = (a > b) ? a : b;
      m = (ab > m) ? ab : m;
      o += overflow_of(v[k].x, cap) + overflow_of(v[k].y, cap) + overflow_of(v[k].z, cap) +
           overflow_of(v[k].w, cap);
    }
  }
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * NT;
  for (uint64_t j = 4u * nvec + static_cast<uint64_t>(blockIdx.x) * NT + threadIdx.x; j < cells;
       j += stride) {
    const uint32_t v = conteos[j];
    m = (v > m) ? v : m;
    o += overflow_of(v, cap);
  }
  m = wave_max_u32(m);
  o = wave_add_u32(o);
  if ((threadIdx.x & 63) == 0) {
    s_m[threadIdx.x >> 6] = m;
    s_o[threadIdx.x >> 6] = o;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t bm = 0, bo = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      bm = (s_m[w] > bm) ? s_m[w] : bm;
      bo += s_o[w];
    }
    // the pair goes out with a device-coherent store and has completed
    // before the ticket is taken, so the workgroup that takes the last
    // ticket reads every pair with device-coherent loads (no cache
    // writeback or invalidation, which a release or acquire at device scope
    // would do for every line of the XCD's L2)
    __hip_atomic_store(reinterpret_cast<uint64_t*>(part) + blockIdx.x,
                       static_cast<uint64_t>(bm) | (static_cast<uint64_t>(bo) << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(kWaitLoadsAndStores);
    const uint32_t t = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (t == gridDim.x - 1u) ? 1u : 0u;
  }
  __syncthreads();
  if (s_last == 0u) return;  // workgroup-uniform
  uint2 pr = make_uint2(0u, 0u);
  if (threadIdx.x < gridDim.x) {
    const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t*>(part) + threadIdx.x, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    pr = make_uint2(static_cast<uint32_t>(v), static_cast<uint32_t>(v >> 32));
  }
  m = wave_max_u32(pr.x);
  o = wave_add_u32(pr.y);
  __syncthreads();  // s_m/s_o reads of the fold above are done
  if ((threadIdx.x & 63) == 0) {
    s_m[threadIdx.x >> 6] = m;
    s_o[threadIdx.x >> 6] = o;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t bm = 0, bo = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      bm = (s_m[w] > bm) ? s_m[w] : bm;
      bo += s_o[w];
    }
    diag[0] = bm;
    diag[1] = bo;
    __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next launch
  }
}

}  // namespace ugp
