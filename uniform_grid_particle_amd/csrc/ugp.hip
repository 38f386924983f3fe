// ugp.hip -- uniform-grid particle index build for MI355X (gfx950, CDNA4).
//
// Kernels and the C ABI declared in include/ugp.h. The build is a counting
// sort by cell key:
//   clear   zero conteos and the per-tile partial sums
//   count   cell key -> celdaDe, histogram -> conteos, per-tile sums
//   scan    conteos -> inicios (exclusive, total in the extra slot) and the
//           scatter cursor (a copy of inicios)
//   scatter cursor atomics -> ordenado, and (default) the record itself
//   [stable] sort every cell's slice of ordenado ascending
//   [gather] reordered[k] = particles[ordenado[k]]
//
// Source pages (titles and sections): "Contar partículas por celda" (El
// kernel; La contención de las celdas densas), "Construir el índice de la
// rejilla con un prefix sum" (Del conteo al inicio; La dispersión; La cadena
// completa; El orden dentro de la celda), "Reordenar por celda y la
// coalescencia de memoria" (El kernel de reordenación; El orden de las
// celdas también importa), "El estado de las partículas en storage
// buffers" (La estructura y su alineación).
//
// Differences from the pages' WebGPU chain, all result-preserving:
//  * The scan needs no look-back and no multi-level dispatch chain: the
//    count kernel also accumulates, per workgroup in LDS, how many
//    particles fall in each scan tile (a tile is 2^bin_shift consecutive
//    cells, at most 512 tiles), and flushes those partial sums with one
//    global atomic per touched tile. Every scan workgroup then sums the
//    tile totals before its own tile and scans its cells independently.
//  * The scatter cursor is initialised to inicios by the scan (instead of
//    a second clear to zero), so a slot is one returning atomic, and
//    conteos is left holding the histogram.
//  * By default the scatter kernel also moves the 32-byte record to its
//    slot (coalesced read, scattered write) and no separate gather kernel
//    runs; UGP_FLAG_GATHER selects the pages' gather kernel instead.
//  * Stable mode sorts each cell's slice by particle index after the
//    atomic scatter (registers for short cells, LDS bitonic sort for long
//    ones, an ordered compaction for cells beyond the LDS capacity).

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "ugp.h"

namespace {

constexpr int kBlock = 256;          // threads per workgroup (4 waves of 64)
constexpr int kCountItems = 8;       // particles per thread in count / scatter
constexpr int kGatherItems = 8;      // half-records per thread in the gather
constexpr int kScanItems = 16;       // consecutive cells per thread in the scan
constexpr uint32_t kScanSub = kBlock * kScanItems;  // 4096 cells per scan sub-tile
constexpr uint32_t kMaxBins = 512;   // scan tiles (LDS bins in count) upper bound
constexpr uint32_t kMinBinShift = 12;  // a scan tile is at least one sub-tile
constexpr uint32_t kSmallSort = 16;  // cells up to this length are sorted in registers
constexpr int kSortBlock = 1024;     // threads of the long-cell sort
constexpr uint32_t kLdsSort = 16384; // longest cell sorted in LDS (64 KiB)
constexpr int kSortGrid = 512;       // workgroups of the long-cell sort
constexpr uint32_t kMaxDim = 1u << 24;
constexpr uint32_t kCounterWords = 64;  // small counters block after the tile sums

struct GridParams {
  float ox, oy, oz;  // origin
  float h;           // cell size
  float tx, ty, tz;  // dims - 1 as floats (exact: dims <= 2^24)
  uint32_t nx;       // dims[0]
  uint32_t nxy;      // dims[0] * dims[1] (fits: cells < 2^32)
};

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

// Cell along one axis: binary32 subtraction, correctly rounded binary32
// division (this file is built without fast-math, so '/' is the IEEE
// division), floor, then clamp in the float domain before converting.
// The lower test is false for NaN, so NaN and -inf go to 0; +inf and
// everything past the last face go to dim-1.
__device__ __forceinline__ uint32_t axis_cell(float p, float o, float h, float top) {
  const float q = (p - o) / h;
  float f = floorf(q);
  f = (f >= 0.0f) ? f : 0.0f;
  f = (f > top) ? top : f;
  return static_cast<uint32_t>(f);
}

__device__ __forceinline__ uint32_t cell_of(float x, float y, float z, const GridParams& g) {
  const uint32_t kx = axis_cell(x, g.ox, g.h, g.tx);
  const uint32_t ky = axis_cell(y, g.oy, g.h, g.ty);
  const uint32_t kz = axis_cell(z, g.oz, g.h, g.tz);
  return kx + ky * g.nx + kz * g.nxy;  // < cells <= 2^32-2, no wrap
}

__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// Exclusive scan of one value per thread across a workgroup of NT threads.
// Returns the exclusive prefix; *total receives the workgroup sum.
// Contains two barriers; every thread of the workgroup must call it.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t x, uint32_t* s_wave,
                                                        uint32_t* total) {
  constexpr int kWaves = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const uint32_t incl = wave_inclusive_sum(x);
  if (lane == 63) s_wave[wid] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t v = s_wave[w];
    before += (w < wid) ? v : 0u;
    all += v;
  }
  __syncthreads();
  *total = all;
  return before + incl - x;
}

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

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

// Stable mode, short cells: one thread per cell. Cells of at most 16
// entries are sorted in registers with a bitonic network (static indices,
// padding with 0xFFFFFFFF which no particle index reaches); longer cells
// are appended to a list for the LDS kernel.
__global__ __launch_bounds__(kBlock) void sort_short_cells_kernel(
    const uint32_t* __restrict__ inicios, uint32_t cells, uint32_t n,
    uint32_t* __restrict__ ordenado, uint32_t* __restrict__ long_list, uint32_t long_cap,
    uint32_t* __restrict__ long_count) {
  const uint32_t c = blockIdx.x * kBlock + threadIdx.x;
  if (c >= cells) return;
  const uint32_t s = inicios[c];
  const uint32_t e = inicios[c + 1];
  if (e > n || e <= s || e - s < 2) return;
  const uint32_t len = e - s;
  if (len > kSmallSort) {
    const uint32_t k = atomicAdd(long_count, 1u);
    if (k < long_cap) long_list[k] = c;
    return;
  }
  uint32_t v[kSmallSort];
#pragma unroll
  for (uint32_t k = 0; k < kSmallSort; ++k) v[k] = (k < len) ? ordenado[s + k] : 0xFFFFFFFFu;
#pragma unroll
  for (uint32_t kk = 2; kk <= kSmallSort; kk <<= 1) {
#pragma unroll
    for (uint32_t j = kk >> 1; j > 0; j >>= 1) {
#pragma unroll
      for (uint32_t i = 0; i < kSmallSort; ++i) {
        const uint32_t l = i ^ j;
        if (l > i) {
          const bool up = (i & kk) == 0;
          const uint32_t a = v[i], b = v[l];
          if ((a > b) == up) {
            v[i] = b;
            v[l] = a;
          }
        }
      }
    }
  }
#pragma unroll
  for (uint32_t k = 0; k < kSmallSort; ++k)
    if (k < len) ordenado[s + k] = v[k];
}

// Stable mode, long cells: one workgroup per listed cell (grid-stride over
// the list). Up to 16384 entries: bitonic sort in LDS. Longer: ordered
// compaction, i.e. walk all particles in index order and append those of
// this cell (the cell's membership is exact already; only order changes).
__global__ __launch_bounds__(kSortBlock) void sort_long_cells_kernel(
    const uint32_t* __restrict__ inicios, const uint32_t* __restrict__ celdaDe, uint32_t n,
    const uint32_t* __restrict__ long_list, uint32_t long_cap,
    const uint32_t* __restrict__ long_count, uint32_t* __restrict__ ordenado) {
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
      for (uint32_t t = threadIdx.x; t < len; t += kSortBlock) ordenado[s + t] = s_keys[t];
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
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline uint32_t ceil_log2_u64(uint64_t x) {
  uint32_t s = 0;
  while ((1ull << s) < x) ++s;
  return s;
}

struct Plan {
  uint64_t cells = 0;
  uint32_t bin_shift = kMinBinShift;
  uint32_t nbins = 1;
  uint32_t long_cap = 0;
  size_t off_cursor = 0;
  size_t off_small = 0;  // tile sums (nbins words) then kCounterWords counters
  size_t off_long = 0;
  size_t total = 0;
};

int make_plan(uint32_t n, const uint32_t dims[3], uint32_t flags, Plan* p) {
  if (!dims) return UGP_ERR_NULL;
  if (flags & ~(UGP_FLAG_STABLE | UGP_FLAG_GATHER)) return UGP_ERR_ARG;
  for (int a = 0; a < 3; ++a)
    if (dims[a] < 1u || dims[a] > kMaxDim) return UGP_ERR_RANGE;
  const uint64_t cells = static_cast<uint64_t>(dims[0]) * dims[1] * dims[2];
  if (cells > 0xFFFFFFFEull) return UGP_ERR_RANGE;
  p->cells = cells;
  const uint32_t lg = ceil_log2_u64(cells);
  p->bin_shift = (lg > kMinBinShift + 9) ? lg - 9 : kMinBinShift;
  p->nbins = static_cast<uint32_t>((cells + (1ull << p->bin_shift) - 1) >> p->bin_shift);
  size_t off = 0;
  p->off_cursor = off;
  off = align_up(off + cells * 4u, 256);
  p->off_small = off;
  off = align_up(off + (static_cast<size_t>(p->nbins) + kCounterWords) * 4u, 256);
  p->off_long = off;
  if (flags & UGP_FLAG_STABLE) {
    const uint64_t cap = static_cast<uint64_t>(n) / (kSmallSort + 1) + 1;
    p->long_cap = static_cast<uint32_t>(cap < cells ? cap : cells);
    off = align_up(off + static_cast<size_t>(p->long_cap) * 4u, 256);
  }
  p->total = off;
  return UGP_OK;
}

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(const Span& a, const Span& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct BuildArgs {
  const ugp_particle* particles;
  uint32_t n;
  const float* origin;
  float cell_size;
  const uint32_t* dims;
  uint32_t* celdaDe;
  uint32_t* conteos;
  uint32_t* inicios;
  uint32_t* ordenado;
  ugp_particle* reordered;
  void* workspace;
  size_t workspace_bytes;
  uint32_t flags;
  hipStream_t stream;
};

int validate(const BuildArgs& a, Plan* plan) {
  if (!a.origin || !a.dims) return UGP_ERR_NULL;
  int st = make_plan(a.n, a.dims, a.flags, plan);
  if (st != UGP_OK) return st;
  if (!std::isfinite(a.cell_size) || !(a.cell_size >= FLT_MIN)) return UGP_ERR_ARG;
  for (int k = 0; k < 3; ++k)
    if (!std::isfinite(a.origin[k])) return UGP_ERR_ARG;
  if (!a.conteos || !a.inicios || !a.workspace) return UGP_ERR_NULL;
  if (a.n > 0 && (!a.particles || !a.celdaDe || !a.ordenado || !a.reordered)) return UGP_ERR_NULL;
  if (!aligned(a.conteos, 16) || !aligned(a.inicios, 16) || !aligned(a.workspace, 256))
    return UGP_ERR_ALIGN;
  if (a.n > 0 && (!aligned(a.particles, 16) || !aligned(a.reordered, 16) ||
                  !aligned(a.celdaDe, 16) || !aligned(a.ordenado, 16)))
    return UGP_ERR_ALIGN;
  if (a.workspace_bytes < plan->total) return UGP_ERR_WORKSPACE;
  const size_t n = a.n;
  const size_t c = plan->cells;
  const Span spans[7] = {
      {reinterpret_cast<uintptr_t>(a.particles), reinterpret_cast<uintptr_t>(a.particles) + 32 * n},
      {reinterpret_cast<uintptr_t>(a.celdaDe), reinterpret_cast<uintptr_t>(a.celdaDe) + 4 * n},
      {reinterpret_cast<uintptr_t>(a.conteos), reinterpret_cast<uintptr_t>(a.conteos) + 4 * c},
      {reinterpret_cast<uintptr_t>(a.inicios), reinterpret_cast<uintptr_t>(a.inicios) + 4 * (c + 1)},
      {reinterpret_cast<uintptr_t>(a.ordenado), reinterpret_cast<uintptr_t>(a.ordenado) + 4 * n},
      {reinterpret_cast<uintptr_t>(a.reordered), reinterpret_cast<uintptr_t>(a.reordered) + 32 * n},
      {reinterpret_cast<uintptr_t>(a.workspace), reinterpret_cast<uintptr_t>(a.workspace) + plan->total},
  };
  for (int i = 0; i < 7; ++i)
    for (int j = i + 1; j < 7; ++j)
      if (overlap(spans[i], spans[j])) return UGP_ERR_ALIAS;
  return UGP_OK;
}

GridParams grid_params(const BuildArgs& a) {
  GridParams g;
  g.ox = a.origin[0];
  g.oy = a.origin[1];
  g.oz = a.origin[2];
  g.h = a.cell_size;
  g.tx = static_cast<float>(a.dims[0] - 1u);
  g.ty = static_cast<float>(a.dims[1] - 1u);
  g.tz = static_cast<float>(a.dims[2] - 1u);
  g.nx = a.dims[0];
  g.nxy = a.dims[0] * a.dims[1];
  return g;
}

inline uint32_t blocks_for(uint64_t work, uint64_t per_block) {
  return static_cast<uint32_t>((work + per_block - 1) / per_block);
}

int enqueue_stage(uint32_t stage, const BuildArgs& a, const Plan& p) {
  char* ws = static_cast<char*>(a.workspace);
  uint32_t* cursor = reinterpret_cast<uint32_t*>(ws + p.off_cursor);
  uint32_t* tilesum = reinterpret_cast<uint32_t*>(ws + p.off_small);
  uint32_t* counters = tilesum + p.nbins;
  uint32_t* long_list = reinterpret_cast<uint32_t*>(ws + p.off_long);
  const bool stable = (a.flags & UGP_FLAG_STABLE) != 0;
  const bool gather = stable || (a.flags & UGP_FLAG_GATHER) != 0;
  const uint32_t n = a.n;
  const uint32_t cells = static_cast<uint32_t>(p.cells);
  hipStream_t s = a.stream;
  switch (stage) {
    case UGP_STAGE_CLEAR: {
      uint64_t vec = p.cells / 4;
      uint32_t blocks = blocks_for(vec ? vec : 1, kBlock);
      if (blocks > 2048) blocks = 2048;
      hipLaunchKernelGGL(clear_kernel, dim3(blocks), dim3(kBlock), 0, s, a.conteos, p.cells,
                         tilesum, p.nbins + kCounterWords);
      break;
    }
    case UGP_STAGE_COUNT: {
      if (n == 0) return UGP_OK;
      hipLaunchKernelGGL(count_kernel, dim3(blocks_for(n, kBlock * kCountItems)), dim3(kBlock), 0, s,
                         reinterpret_cast<const float4*>(a.particles), n, grid_params(a),
                         a.celdaDe, a.conteos, tilesum, p.bin_shift, p.nbins);
      break;
    }
    case UGP_STAGE_SCAN: {
      hipLaunchKernelGGL(scan_kernel, dim3(p.nbins), dim3(kBlock), 0, s, a.conteos, p.cells,
                         tilesum, p.bin_shift, a.inicios, n ? cursor : nullptr);
      break;
    }
    case UGP_STAGE_SCATTER: {
      if (n == 0) return UGP_OK;
      const dim3 grid(blocks_for(n, kBlock * kCountItems));
      if (gather) {
        hipLaunchKernelGGL(scatter_kernel<false>, grid, dim3(kBlock), 0, s, a.celdaDe, n, cells,
                           cursor, a.ordenado, nullptr, nullptr);
      } else {
        hipLaunchKernelGGL(scatter_kernel<true>, grid, dim3(kBlock), 0, s, a.celdaDe, n, cells,
                           cursor, a.ordenado, reinterpret_cast<const uint4*>(a.particles),
                           reinterpret_cast<uint4*>(a.reordered));
      }
      break;
    }
    case UGP_STAGE_SORT_CELLS: {
      if (!stable || n < 2) return UGP_OK;
      hipLaunchKernelGGL(sort_short_cells_kernel, dim3(blocks_for(cells, kBlock)), dim3(kBlock), 0,
                         s, a.inicios, cells, n, a.ordenado, long_list, p.long_cap, counters);
      hipLaunchKernelGGL(sort_long_cells_kernel, dim3(kSortGrid), dim3(kSortBlock), 0, s, a.inicios,
                         a.celdaDe, n, long_list, p.long_cap, counters, a.ordenado);
      break;
    }
    case UGP_STAGE_GATHER: {
      if (!gather || n == 0) return UGP_OK;
      hipLaunchKernelGGL(gather_kernel, dim3(blocks_for(n, kBlock * kGatherItems / 2)), dim3(kBlock),
                         0, s, a.ordenado, n, n, reinterpret_cast<const uint4*>(a.particles),
                         reinterpret_cast<uint4*>(a.reordered));
      break;
    }
    default:
      return UGP_ERR_ARG;
  }
  return hipGetLastError() == hipSuccess ? UGP_OK : UGP_ERR_HIP;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

extern "C" {

int ugp_abi_version(void) { return 1; }

const char* ugp_status_string(int status) {
  switch (status) {
    case UGP_OK: return "ok";
    case UGP_ERR_NULL: return "a required pointer is NULL";
    case UGP_ERR_ARG: return "invalid argument (cell_size, origin, flags or stage)";
    case UGP_ERR_RANGE: return "grid dimensions out of range (each dim in [1, 2^24], cells <= 2^32-2)";
    case UGP_ERR_ALIAS: return "two buffers overlap";
    case UGP_ERR_ALIGN: return "misaligned buffer (arrays need 16-byte, workspace 256-byte alignment)";
    case UGP_ERR_WORKSPACE: return "workspace too small";
    case UGP_ERR_HIP: return "HIP runtime error while enqueueing";
    default: return "unknown status";
  }
}

int ugp_grid_workspace_bytes(uint32_t n, const uint32_t dims[3], uint32_t flags, size_t* bytes) {
  if (!bytes) return UGP_ERR_NULL;
  Plan p;
  const int st = make_plan(n, dims, flags, &p);
  if (st != UGP_OK) return st;
  *bytes = p.total;
  return UGP_OK;
}

int ugp_grid_build_stage(uint32_t stage, const ugp_particle* particles, uint32_t n,
                         const float origin[3], float cell_size, const uint32_t dims[3],
                         uint32_t* celdaDe, uint32_t* conteos, uint32_t* inicios,
                         uint32_t* ordenado, ugp_particle* reordered, void* workspace,
                         size_t workspace_bytes, uint32_t flags, void* stream) {
  if (stage >= UGP_NUM_STAGES) return UGP_ERR_ARG;
  const BuildArgs a{particles, n, origin, cell_size, dims, celdaDe, conteos, inicios, ordenado,
                    reordered, workspace, workspace_bytes, flags,
                    static_cast<hipStream_t>(stream)};
  Plan p;
  const int st = validate(a, &p);
  if (st != UGP_OK) return st;
  return enqueue_stage(stage, a, p);
}

int ugp_grid_build(const ugp_particle* particles, uint32_t n, const float origin[3],
                   float cell_size, const uint32_t dims[3], uint32_t* celdaDe, uint32_t* conteos,
                   uint32_t* inicios, uint32_t* ordenado, ugp_particle* reordered, void* workspace,
                   size_t workspace_bytes, uint32_t flags, void* stream) {
  const BuildArgs a{particles, n, origin, cell_size, dims, celdaDe, conteos, inicios, ordenado,
                    reordered, workspace, workspace_bytes, flags,
                    static_cast<hipStream_t>(stream)};
  Plan p;
  int st = validate(a, &p);
  if (st != UGP_OK) return st;
  for (uint32_t stage = 0; stage < UGP_NUM_STAGES; ++stage) {
    st = enqueue_stage(stage, a, p);
    if (st != UGP_OK) return st;
  }
  return UGP_OK;
}

int ugp_scan_workspace_bytes(uint32_t count, size_t* bytes) {
  if (!bytes) return UGP_ERR_NULL;
  const uint64_t c = count ? count : 1;
  const uint32_t lg = ceil_log2_u64(c);
  const uint32_t shift = (lg > kMinBinShift + 9) ? lg - 9 : kMinBinShift;
  const uint64_t nbins = (c + (1ull << shift) - 1) >> shift;
  *bytes = align_up(nbins * 4u, 256);
  return UGP_OK;
}

int ugp_exclusive_scan_u32(const uint32_t* in, uint32_t count, uint32_t* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!out || !workspace || (count > 0 && !in)) return UGP_ERR_NULL;
  if (!aligned(out, 16) || (count > 0 && !aligned(in, 16)) || !aligned(workspace, 256))
    return UGP_ERR_ALIGN;
  size_t need = 0;
  ugp_scan_workspace_bytes(count, &need);
  if (workspace_bytes < need) return UGP_ERR_WORKSPACE;
  const Span si{reinterpret_cast<uintptr_t>(in), reinterpret_cast<uintptr_t>(in) + 4ull * count};
  const Span so{reinterpret_cast<uintptr_t>(out), reinterpret_cast<uintptr_t>(out) + 4ull * (count + 1ull)};
  const Span sw{reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need};
  if (overlap(si, so) || overlap(si, sw) || overlap(so, sw)) return UGP_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* tilesum = static_cast<uint32_t*>(workspace);
  if (count == 0) {
    // out[0] = 0: a one-word clear.
    hipLaunchKernelGGL(clear_kernel, dim3(1), dim3(kBlock), 0, s, out, 1ull, nullptr, 0u);
    return hipGetLastError() == hipSuccess ? UGP_OK : UGP_ERR_HIP;
  }
  const uint32_t lg = ceil_log2_u64(count);
  const uint32_t shift = (lg > kMinBinShift + 9) ? lg - 9 : kMinBinShift;
  const uint32_t nbins = static_cast<uint32_t>((static_cast<uint64_t>(count) + (1ull << shift) - 1) >> shift);
  hipLaunchKernelGGL(tile_reduce_kernel, dim3(nbins), dim3(kBlock), 0, s, in,
                     static_cast<uint64_t>(count), shift, tilesum);
  hipLaunchKernelGGL(scan_kernel, dim3(nbins), dim3(kBlock), 0, s, in, static_cast<uint64_t>(count),
                     tilesum, shift, out, nullptr);
  return hipGetLastError() == hipSuccess ? UGP_OK : UGP_ERR_HIP;
}

int ugp_reorder(const ugp_particle* src, uint32_t n_src, const uint32_t* idx, uint32_t n,
                ugp_particle* dst, void* stream) {
  if (n == 0) return UGP_OK;
  if (!src || !idx || !dst) return UGP_ERR_NULL;
  if (!aligned(src, 16) || !aligned(dst, 16) || !aligned(idx, 4)) return UGP_ERR_ALIGN;
  const Span ss{reinterpret_cast<uintptr_t>(src), reinterpret_cast<uintptr_t>(src) + 32ull * n_src};
  const Span si{reinterpret_cast<uintptr_t>(idx), reinterpret_cast<uintptr_t>(idx) + 4ull * n};
  const Span sd{reinterpret_cast<uintptr_t>(dst), reinterpret_cast<uintptr_t>(dst) + 32ull * n};
  if (overlap(ss, sd) || overlap(si, sd)) return UGP_ERR_ALIAS;
  if (n_src == 0) return UGP_OK;  // every index is out of range: nothing to write
  hipLaunchKernelGGL(gather_kernel, dim3(blocks_for(n, kBlock * kGatherItems / 2)), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), idx, n, n_src,
                     reinterpret_cast<const uint4*>(src), reinterpret_cast<uint4*>(dst));
  return hipGetLastError() == hipSuccess ? UGP_OK : UGP_ERR_HIP;
}

}  // extern "C"
