// common.h -- constants and device helpers shared by the index-build kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

namespace ugp {

// Kernel launches of the library. When a timed build has armed a pair of
// events (ugp_grid_build_timed), the next launch records them at that
// kernel's own start and end (so the interval is the kernel alone, as a
// profiler's kernel trace measures it) and disarms them; otherwise a plain
// launch. Host-side, per calling thread.
struct TimedLaunch {
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local TimedLaunch g_timed_launch;

template <typename F, typename... Args>
inline void launch(F kernel, const dim3& grid, const dim3& block, uint32_t shmem, hipStream_t s, Args... args) {
  if (g_timed_launch.start != nullptr) {
    const TimedLaunch t = g_timed_launch;
    g_timed_launch = TimedLaunch{};
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, t.start, t.stop, 0u, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
  }
}

constexpr int kBlock = 256;     // threads of the streaming kernels (4 waves of 64)
constexpr uint32_t kMaxDim = 1u << 24;
// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left free (CDNA
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitLoadsAndStores = 0x0F70;

// Stable mode on the tile paths: the cells a tile kernel leaves in arrival
// order. Cells of 2..kRankSortMax particles go on the short list (put in
// order afterwards by one wave each), longer ones on the long list (one
// workgroup each). One block of words holds both: the two list lengths
// (zeroed by the first kernel of the build) at base[0] and base[1], the
// short list from base[kFixHeader], the long list after it. A list never
// holds more than its capacity.
constexpr uint32_t kRankSortMax = 256;
constexpr uint32_t kFixHeader = 64;  // words before the short list (256 bytes)
struct FixLists {
  uint32_t* base;
  uint32_t fix_cap;   // short-list capacity
  uint32_t long_cap;  // long-list capacity
  __device__ __forceinline__ uint32_t* counts() const { return base; }
  __device__ __forceinline__ uint32_t* fix() const { return base + kFixHeader; }
  __device__ __forceinline__ uint32_t* lng() const { return base + kFixHeader + fix_cap; }
  // one word per output place: the arrival-order index, written by the tile
  // kernel for every tile that holds a long cell or overflows its staging,
  // so the long-cell fix-up reads the cell's indices from a copy it does not
  // itself rewrite
  __device__ __forceinline__ uint32_t* idx() const { return base + kFixHeader + fix_cap + long_cap; }
};

// Work shared among the workgroups of one tile kernel launch: the scatter
// of tiles past the staged capacity. The workgroup that owns such a tile
// claims one of kMaxSlots slots as soon as it knows its count; while it
// counts the tile it writes the chunk-array position of every particle of
// the tile, in the tile's own order, into the tile's places of a source
// list (n words) -- or, when every chunk run of the tile is short, it
// leaves the tile's run table in the slot instead, from which a round
// rebuilds those positions; after the scan it leaves one cursor per cell in
// the slot (its next free tile-local place) and marks the slot ready. The tile's
// particles are then scattered in rounds of kRound, each taken from the
// slot's ticket by the owner or by any other tile's workgroup that saw a
// claimed slot before its own stores. A workgroup waits only for a slot that
// was claimed, i.e. for an owner that is running and that waits for no one.
//   header (kQueueHeader words, zeroed by the first kernel of the build):
//     [0] slots claimed; for slot s: [kReadyWord + s] ready (0/1),
//     [kTicketWord + s] next round to hand out, [kRoundsWord + s] rounds,
//     [kStartWord + s] the tile's first place, [kCountWord + s] its count,
//     [kTileWord + s] the tile (| kRunTableBit: the run table holds the sources)
//   slot s: one cursor per cell of a tile, then the run table (kQueueRunWords)
constexpr uint32_t kRound = 4096;
constexpr uint32_t kMaxSlots = 64;
constexpr uint32_t kReadyWord = 64;
constexpr uint32_t kTicketWord = kReadyWord + kMaxSlots;
constexpr uint32_t kRoundsWord = kTicketWord + kMaxSlots;
constexpr uint32_t kStartWord = kRoundsWord + kMaxSlots;
constexpr uint32_t kCountWord = kStartWord + kMaxSlots;
constexpr uint32_t kTileWord = kCountWord + kMaxSlots;
constexpr uint32_t kQueueHeader = kTileWord + kMaxSlots;
// chunk_sort's index words on the staged path: (tile-local cell << kIdxBits)
// | index inside the chunk (chunks of at most 2^kIdxBits particles)
constexpr uint32_t kIdxBits = 11;
// A slot also holds a run table (kQueueRunWords words after its cursors):
// the tile-local start of each chunk's run, then where each run starts in
// the chunk arrays, written instead of the source list when every run of
// the tile is short (the rounds rebuild their sources from it).
constexpr uint32_t kQueueRunWords = 2048;
constexpr uint32_t kRunTableBit = 0x80000000u;  // in a slot's tile word: its rounds use the run table
struct TileQueue {
  uint32_t* base;      // nullptr: no sharing (single-tile path)
  uint32_t* sources;   // n words: chunk-array positions of shared tiles' particles
  uint32_t slot_words; // words per slot: one cursor per cell of a tile, then the run table
  uint32_t run_off;    // where the run table starts in a slot (the tile size)
  __device__ __forceinline__ uint32_t* hdr() const { return base; }
  __device__ __forceinline__ uint32_t* cursors(uint32_t s) const {
    return base + kQueueHeader + static_cast<size_t>(s) * slot_words;
  }
  __device__ __forceinline__ uint32_t* runs(uint32_t s) const { return cursors(s) + run_off; }
};

struct GridParams {
  float ox, oy, oz;  // origin
  float h;           // cell size
  float tx, ty, tz;  // dims - 1 as floats (exact: dims <= 2^24)
  uint32_t nx;       // dims[0]
  uint32_t nxy;      // dims[0] * dims[1] (fits: cells < 2^32)
  uint32_t morton;   // 1: cells numbered along the Z curve, 0: linearly
};

// Cell along one axis: binary32 subtraction, correctly rounded binary32
// division (the library is built without fast-math, so '/' is the IEEE
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

// Spreads the low 10 bits of v to bit positions 0, 3, 6, ..., 27 (each
// step moves the upper half of every group to a slot three times wider).
__device__ __forceinline__ uint32_t spread_bits3(uint32_t v) {
  v &= 0x3FFu;
  v = (v | (v << 16)) & 0x030000FFu;
  v = (v | (v << 8)) & 0x0300F00Fu;
  v = (v | (v << 4)) & 0x030C30C3u;
  v = (v | (v << 2)) & 0x09249249u;
  return v;
}

// Cell key of a position. Linear: x + y*nx + z*nx*ny (< cells <= 2^32-2,
// no wrap). Morton (page "Reordenar por celda y la coalescencia de
// memoria", section "El orden de las celdas también importa"): bit b of
// x, y, z at key bits 3b, 3b+1, 3b+2 (coordinates < 2^10 on such grids).
// g.morton is the same for every thread, so the branch is uniform.
__device__ __forceinline__ uint32_t cell_of(float x, float y, float z, const GridParams& g) {
  const uint32_t kx = axis_cell(x, g.ox, g.h, g.tx);
  const uint32_t ky = axis_cell(y, g.oy, g.h, g.ty);
  const uint32_t kz = axis_cell(z, g.oz, g.h, g.tz);
  if (g.morton) return spread_bits3(kx) | (spread_bits3(ky) << 1) | (spread_bits3(kz) << 2);
  return kx + ky * g.nx + kz * g.nxy;
}

// Streaming accesses: data read or written once by this kernel. The
// non-temporal hint keeps it from displacing reused lines in the caches.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(uint4* p, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ uint32_t load_stream(const uint32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_stream(uint32_t* p, uint32_t v) { __builtin_nontemporal_store(v, p); }

// Stores written through the L2 to memory (cache policy sc1: device scope),
// through a buffer resource over one workgroup's own output range of `bytes`
// bytes (the hardware drops a store past them; offsets are from the range's
// start). A workgroup's dirty L2 lines are otherwise written back when the
// kernel ends, after its last store: sent out while it runs, they leave that
// write-back short. Used for the chunk kernel's chunk array when it is larger
// than the L2 caches hold (the next kernel reads it from memory either way)
// and for the tile kernel's conteos and inicios (never read again by the
// build). Measured on MI355X, each change against the one before:
//   conteos and inicios  Sparse 21.9 -> 20.7 us, Large 860 -> 843 us,
//                        Baseline unchanged;
//   the chunk array      Baseline 37.4 -> 36.5 us, Sparse 20.6 -> 20.1 us,
//                        Large 842 -> 835 us.
// Written through, the tile kernel's records (its last stores) cost 4 us at
// Baseline and celdaDe gained nothing.
constexpr int kStoreThrough = 16;  // the sc1 bit of a buffer store's cache policy
constexpr int kStoreThroughNT = 16 | 2;  // sc1 and the non-temporal bit
__device__ __forceinline__ __amdgpu_buffer_rsrc_t output_rsrc(void* p, uint32_t bytes) {
  // dword 3: 32-bit data format, no swizzle, no thread-id offset
  return __builtin_amdgcn_make_buffer_rsrc(p, static_cast<short>(0), static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ void store_through(__amdgpu_buffer_rsrc_t r, uint32_t offset, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, static_cast<int>(offset), 0, kStoreThrough);
}
__device__ __forceinline__ void store_through(__amdgpu_buffer_rsrc_t r, uint32_t offset, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, static_cast<int>(offset), 0, kStoreThrough);
}
// The same with the non-temporal bit as well (the bucketed path's coarse
// sort: Large 835 -> 808 us measured; on the staged path it costs 1.3 us).
__device__ __forceinline__ void store_through_nt(__amdgpu_buffer_rsrc_t r, uint32_t offset, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, static_cast<int>(offset), 0, kStoreThroughNT);
}
__device__ __forceinline__ void store_through_nt(__amdgpu_buffer_rsrc_t r, uint32_t offset, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, static_cast<int>(offset), 0, kStoreThroughNT);
}

// Inclusive prefix sum across the 64 lanes of a wave, with DPP lane moves
// (no LDS traffic): shifts of 1, 2, 4 and 8 lanes inside each row of 16
// give row-inclusive sums, then row 0's total is broadcast into row 1 and
// row 2's into row 3 (row_bcast:15), then the total of rows 0-1 into rows
// 2-3 (row_bcast:31). Lanes without a source add 0.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
  constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
  constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowShr1, 0xf, 0xf, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowShr2, 0xf, 0xf, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowShr4, 0xf, 0xf, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowShr8, 0xf, 0xf, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowBcast15, 0xa, 0xf, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowBcast31, 0xc, 0xf, false));
  return x;
}

// Inclusive maximum across the 64 lanes of a wave (same DPP moves as
// wave_inclusive_sum; lanes without a source take 0, the identity for the
// unsigned values it is used on).
__device__ __forceinline__ uint32_t wave_inclusive_max(uint32_t x) {
  constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
  constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
  uint32_t y;
  y = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowShr1, 0xf, 0xf, false));
  x = (y > x) ? y : x;
  y = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowShr2, 0xf, 0xf, false));
  x = (y > x) ? y : x;
  y = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowShr4, 0xf, 0xf, false));
  x = (y > x) ? y : x;
  y = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowShr8, 0xf, 0xf, false));
  x = (y > x) ? y : x;
  y = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowBcast15, 0xa, 0xf, false));
  x = (y > x) ? y : x;
  y = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kRowBcast31, 0xc, 0xf, false));
  x = (y > x) ? y : x;
  return x;
}

// Exclusive maximum of one value per thread across a workgroup of NT
// threads (0 for thread 0). s_wave: NT/64 words of LDS; two barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_max(uint32_t x, uint32_t* s_wave) {
  constexpr int kWaves = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const uint32_t incl = wave_inclusive_max(x);
  if (lane == 63) s_wave[wid] = incl;
  const uint32_t up = static_cast<uint32_t>(__shfl_up(static_cast<int>(incl), 1, 64));
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t v = s_wave[w];
    before = (w < wid && v > before) ? v : before;
  }
  __syncthreads();
  const uint32_t in_wave = (lane > 0) ? up : 0u;
  return (in_wave > before) ? in_wave : before;
}

// Exclusive scan of one value per thread across a workgroup of NT threads.
// Returns the exclusive prefix; *total receives the workgroup sum.
// s_wave: NT/64 words of LDS. Contains two barriers; every thread of the
// workgroup must call it.
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

// Maximum of one value per thread across a workgroup (all threads get it).
// s_wave: NT/64 words of LDS; two barriers, every thread must call it.
template <int NT>
__device__ __forceinline__ uint32_t block_max(uint32_t x, uint32_t* s_wave) {
  constexpr int kWaves = NT / 64;
  const uint32_t incl = wave_inclusive_max(x);
  if ((threadIdx.x & 63) == 63) s_wave[threadIdx.x >> 6] = incl;
  __syncthreads();
  uint32_t m = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) m = (s_wave[w] > m) ? s_wave[w] : m;
  __syncthreads();
  return m;
}

// Sum of one value per thread across a workgroup (all threads get it).
template <int NT>
__device__ __forceinline__ uint32_t block_sum(uint32_t x, uint32_t* s_wave) {
  uint32_t total;
  (void)block_exclusive_sum<NT>(x, s_wave, &total);
  return total;
}

}  // namespace ugp
