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

constexpr int kDiagBlock = 256;
constexpr uint32_t kDiagMaxGrid = 1024;

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

// Standalone: diag[0] = max conteos[c], diag[1] += sum max(0, conteos[c] - cap)
// over c < cells. diag must be zeroed before. conteos 16-byte aligned. Each
// thread issues kDiagItems 16-byte loads per round before using any of them.
constexpr int kDiagItems = 4;
// NT threads per workgroup (a template, so that every translation unit that
// sees this header may define it).
template <int NT>
__global__ __launch_bounds__(NT) void diag_kernel(const uint32_t* __restrict__ conteos, uint32_t cells,
                                                  uint32_t cap, uint32_t* __restrict__ diag) {
  __shared__ uint32_t s_m[NT / 64], s_o[NT / 64];
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
  publish_diag<NT>(s_m, s_o, diag);
}

}  // namespace ugp
