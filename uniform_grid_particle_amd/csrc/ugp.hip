// ugp.hip -- uniform-grid particle index build for MI355X (gfx950, CDNA4):
// host side and the C ABI declared in include/ugp.h.
//
// The build is a counting sort of particles by cell key (page "Contar
// partículas por celda", opening paragraph and section "El kernel"):
// count per cell, exclusive scan with a trailing total (page "Construir el
// índice de la rejilla con un prefix sum", section "Del conteo al inicio"),
// scatter of particle indices into each cell's range (same page, section
// "La dispersión"), and a 32-byte record reorder into a second buffer
// (page "Reordenar por celda y la coalescencia de memoria", section "El
// kernel de reordenación").
//
// Five execution paths, chosen on the host from n and the grid size:
//   empty   n == 0: conteos and inicios are zeroed.
//   single  n <= 8192 and keys <= 2^14: the tile kernel alone, one
//           workgroup reading the input directly (one launch).
//   staged  keys <= 2^22 (2^23 on dense grids) and n <= 2^21: the
//           two-kernel, atomic-free counting sort of kernels_staged.h
//           (chunk_sort, tile_sort).
//   bucketed  other grids up to 2^26 keys: the four-kernel atomic-free
//           counting sort of kernels_bucket.h (keys, tile_scan, bucket) ending
//           in the staged tile kernel (tile_sort).
//   direct  larger grids: the global-atomic chain of kernels_direct.h
//           (clear, count, scan, scatter).
// Stable mode (ascending particle index inside every cell): the tile
// kernel orders the cells it can and lists the rest for one fix-up kernel
// (kernels_reorder.h); the direct path orders every cell after its
// scatter. Gather mode adds a gather pass. The overflow
// diagnostics are folded into the staged tile kernel (a compile-time
// variant); the other paths reduce conteos once it is final.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cfloat>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "common.h"
#include "kernels_diag.h"
#include "kernels_neighbor.h"
#include "kernels_direct.h"
#include "kernels_reorder.h"
#include "kernels_staged.h"
#include "kernels_bucket.h"
#include "tile_launch.h"
#include "ugp.h"

namespace ugp {
thread_local TimedLaunch g_timed_launch;
}  // namespace ugp

namespace {

using namespace ugp;

// Library-owned device memory, one copy on every GPU the library runs on,
// zero when the code object loads and held until the process ends. Host
// code never passes these names to a kernel (in host code they stand for a
// host-side shadow, not a device address): it asks for each array's address
// on the current device once (symbol_address) and passes that.
//   diag_scratch  per-workgroup partials and tickets of the one-launch
//                 overflow diagnostics (cell_diag_kernel)
//   scratch       the workspace of ugp_grid_build_noalloc
static __device__ __align__(256) DiagScratch diag_scratch;
static __device__ __align__(256) unsigned char scratch[UGP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_diag_scratch_ptr[kMaxDevices];
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::atomic<uint32_t> g_diag_slot{0};

// Device address of a library-owned __device__ array on the current device:
// hipGetSymbolAddress on the first call per device, the kept address after.
template <typename T>
int symbol_address(const T& symbol, std::atomic<void*>* cache, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return UGP_ERR_HIP;
  void* p = cache[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, symbol) != hipSuccess || p == nullptr) return UGP_ERR_HIP;
    cache[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return UGP_OK;
}

constexpr uint32_t kCounterWords = 64;    // small counter block (direct path)
constexpr uint32_t kMortonMaxBits = 10;   // Morton keys: 10 bits per axis, 2^30 keys

enum class Path { kEmpty, kSingle, kStaged, kBucketed, kDirect };

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline uint32_t ceil_log2_u64(uint64_t x) {
  uint32_t s = 0;
  while ((1ull << s) < x) ++s;
  return s;
}

inline uint32_t blocks_for(uint64_t work, uint64_t per_block) {
  return static_cast<uint32_t>((work + per_block - 1) / per_block);
}

struct Plan {
  Path path = Path::kEmpty;
  uint64_t cells = 0;
  bool stable = false;
  bool gather = false;  // a separate gather kernel moves the records
  bool move = true;     // the scatter kernel itself moves the records
  // tiled
  uint32_t tile_shift = kStagedMinShift, ntiles = 1;
  uint32_t chunk = kChunk;  // particles per chunk_sort workgroup (staged path)
  // bucketed: coarse chunks and buckets (2^cshift keys), row blocks of
  // kRbChunks coarse chunks, [row block x tile] counts, tile and group totals
  uint32_t cshift = 0, nbuckets = 0, ncoarse = 0, nrb = 0, ncount = 0;
  size_t off_rows1 = 0, off_coarse_rec = 0, off_coarse_idx = 0;
  size_t off_hist = 0, off_tile_total = 0, off_group_total = 0;
  // staged
  uint32_t nchunks = 0;
  size_t off_rows = 0, off_chunk_rec = 0, off_chunk_idx = 0;
  // direct
  uint32_t bin_shift = kMinBinShift, nbins = 1;
  size_t off_cursor = 0, off_small = 0;
  // stable
  uint32_t long_cap = 0;
  size_t off_long_count = 0, off_long = 0, off_unstable = 0;
  // stable mode on the tile paths: cells the tile kernel could not sort
  uint32_t fix_cap = 0;
  size_t off_fix = 0;
  // tile paths (staged, bucketed): the shared scatter rounds (TileQueue)
  bool queue = false;
  size_t off_queue = 0, off_sources = 0;
  size_t total = 256;
};

// Bucketed path tile shift: as large as 256 tiles allow but no larger than
// keeps the mean tile at kStagedTarget particles, and at least large enough
// for kBucketMaxTiles tiles (then tiles may exceed the staged capacity; the
// tile kernel takes them in rounds).
uint32_t bucket_shift(uint64_t n, uint64_t cells, uint32_t lg) {
  uint32_t s = (lg > kStagedMinShift + 8) ? lg - 8 : kStagedMinShift;
  uint32_t dense = 0;  // largest d with n * 2^d <= kStagedTarget * cells
  while (dense < 40 && (n << (dense + 1)) <= kStagedTarget * cells) ++dense;
  if (dense < s) s = dense;
  if (s > kStagedMaxShift) s = kStagedMaxShift;  // sparse grids: more, smaller tiles
  const uint32_t fewest = (lg > kStagedMinShift + 12) ? lg - 12 : kStagedMinShift;  // 4096 tiles
  return (s < fewest) ? fewest : s;
}

// The shared scatter of a tile path: the queue header, kMaxSlots slots of
// one cursor per cell of a tile plus a run table, and the source list (n
// words).
size_t plan_queue(Plan* p, uint32_t n, size_t off) {
  p->queue = true;
  p->off_queue = off;
  off = align_up(off + (static_cast<size_t>(kQueueHeader) +
                        static_cast<size_t>(kMaxSlots) * ((1u << p->tile_shift) + kQueueRunWords)) * 4u,
                 256);
  p->off_sources = off;
  return align_up(off + static_cast<size_t>(n) * 4u, 256);
}

int make_plan(uint32_t n, const uint32_t dims[3], uint32_t flags, Plan* p) {
  if (!dims) return UGP_ERR_NULL;
  if (flags & ~(UGP_FLAG_STABLE | UGP_FLAG_GATHER | UGP_FLAG_MORTON | UGP_FLAG_INDEX_ONLY))
    return UGP_ERR_ARG;
  for (int a = 0; a < 3; ++a)
    if (dims[a] < 1u || dims[a] > kMaxDim) return UGP_ERR_RANGE;
  uint64_t cells = static_cast<uint64_t>(dims[0]) * dims[1] * dims[2];
  if (cells > 0xFFFFFFFEull) return UGP_ERR_RANGE;
  if (flags & UGP_FLAG_MORTON) {
    // keys: 2^(3B), 2^B the smallest power of two >= the largest dimension
    uint32_t largest = dims[0] > dims[1] ? dims[0] : dims[1];
    largest = largest > dims[2] ? largest : dims[2];
    const uint32_t bits = ceil_log2_u64(largest);
    if (bits > kMortonMaxBits) return UGP_ERR_RANGE;
    cells = 1ull << (3u * bits);
  }
  *p = Plan{};
  p->cells = cells;
  p->stable = (flags & UGP_FLAG_STABLE) != 0;
  const bool index_only = (flags & UGP_FLAG_INDEX_ONLY) != 0;
  // gather mode writes the records in a pass of their own; stable mode keeps
  // them in the tile kernel (direct path: in a workspace copy that the
  // per-cell sort then permutes into `reordered`)
  p->gather = !index_only && !p->stable && (flags & UGP_FLAG_GATHER) != 0;
  p->move = !index_only && !p->gather;
  const uint32_t lg = ceil_log2_u64(cells);
  size_t off = 0;
  if (n == 0) {
    p->path = Path::kEmpty;
    p->total = 256;
    return UGP_OK;
  }
  // single tile: everything fits one staged tile kernel workgroup
  if (n <= kSingleMax && lg <= kStagedMaxShift) {
    p->path = Path::kSingle;
    p->tile_shift = (lg > kStagedMinShift) ? lg : kStagedMinShift;
    p->ntiles = 1;
    p->nchunks = 1;
  }
  // staged path: tiles of 2^shift consecutive keys. As large as 256 tiles
  // allow (one round of tile_sort workgroups), but no larger than keeps the
  // mean tile at kStagedTarget particles (dense grids: more, smaller tiles),
  // and never more than kStagedMaxTiles tiles.
  uint32_t staged_shift = (lg > kStagedMinShift + 8) ? lg - 8 : kStagedMinShift;
  uint32_t dense_shift = 0;  // largest s with n * 2^s <= kStagedTarget * cells
  while (dense_shift < 40 && (static_cast<uint64_t>(n) << (dense_shift + 1)) <= kStagedTarget * cells)
    ++dense_shift;
  if (dense_shift < staged_shift) staged_shift = dense_shift;
  const uint32_t fewest_shift = (lg > kStagedMinShift + 9) ? lg - 9 : kStagedMinShift;  // 512 tiles
  if (staged_shift < fewest_shift) staged_shift = fewest_shift;
  const uint32_t chunk = (n <= kSmallChunkMaxN) ? kSmallChunk : kChunk;
  const uint64_t nchunks = (static_cast<uint64_t>(n) + chunk - 1) / chunk;
  if (p->path == Path::kSingle) {
    // no workspace beyond the stable-mode lists below
  } else if (staged_shift <= kStagedMaxShift && nchunks <= kStagedMaxChunks) {
    p->path = Path::kStaged;
    p->tile_shift = staged_shift;
    p->ntiles = static_cast<uint32_t>((cells + (1ull << staged_shift) - 1) >> staged_shift);
    p->nchunks = static_cast<uint32_t>(nchunks);
    p->chunk = chunk;
    p->off_rows = off;
    off = align_up(off + static_cast<size_t>(p->nchunks) * p->ntiles * 8u, 256);
    p->off_chunk_rec = off;
    off = align_up(off + static_cast<size_t>(n) * 32u, 256);
    p->off_chunk_idx = off;
    off = align_up(off + static_cast<size_t>(n) * 4u, 256);
    off = plan_queue(p, n, off);
  } else if (bucket_shift(n, cells, lg) <= kStagedMaxShift) {
    // bucketed path: the same tile rule with up to kBucketMaxTiles tiles
    p->path = Path::kBucketed;
    p->tile_shift = bucket_shift(n, cells, lg);
    p->ntiles = static_cast<uint32_t>((cells + (1ull << p->tile_shift) - 1) >> p->tile_shift);
    // buckets of 64 tiles: at most kMaxBuckets, and the bucket-local cell
    // fits the packed index word beside the 11-bit index inside a chunk
    p->cshift = p->tile_shift + 6u;
    static_assert(kStagedMaxShift + 6u + kIdxBits <= 32u, "bucket-local cells fit the packed word");
    static_assert(kBucketMaxTiles <= kMaxBuckets * 64u, "64 tiles per bucket cover every tile");
    static_assert(kMaxBuckets <= kStagedMaxTiles, "buckets fit the chunk kernel's bins");
    p->nbuckets = static_cast<uint32_t>((cells + (1ull << p->cshift) - 1) >> p->cshift);
    p->ncoarse = blocks_for(n, kChunk);
    p->nrb = blocks_for(p->ncoarse, kRbChunks);
    p->ncount = blocks_for(n, kCountPer);
    p->nchunks = 1;  // the tile kernel sees each tile as one contiguous run
    p->off_rows1 = off;
    off = align_up(off + static_cast<size_t>(p->ncoarse) * p->nbuckets * 8u, 256);
    p->off_coarse_rec = off;
    off = align_up(off + static_cast<size_t>(n) * 32u, 256);
    p->off_coarse_idx = off;
    off = align_up(off + static_cast<size_t>(n) * 4u, 256);
    p->off_hist = off;
    off = align_up(off + static_cast<size_t>(p->ncount) * p->ntiles * 4u, 256);
    p->off_tile_total = off;
    off = align_up(off + static_cast<size_t>(p->ntiles) * 4u, 256);
    p->off_group_total = off;
    off = align_up(off + static_cast<size_t>(blocks_for(p->ntiles, 64)) * 4u, 256);
    p->off_rows = off;
    off = align_up(off + static_cast<size_t>(p->ntiles) * 8u, 256);
    p->off_chunk_rec = off;
    off = align_up(off + static_cast<size_t>(n) * 32u, 256);
    p->off_chunk_idx = off;
    off = align_up(off + static_cast<size_t>(n) * 4u, 256);
    off = plan_queue(p, n, off);
  } else {
    p->path = Path::kDirect;
    p->bin_shift = (lg > kMinBinShift + 9) ? lg - 9 : kMinBinShift;
    p->nbins = static_cast<uint32_t>((cells + (1ull << p->bin_shift) - 1) >> p->bin_shift);
    p->off_cursor = off;
    off = align_up(off + cells * 4u, 256);
    p->off_small = off;
    off = align_up(off + (static_cast<size_t>(p->nbins) + kCounterWords) * 4u, 256);
  }
  if (p->stable) {
    // cells longer than kSmallSort (direct path) or kRankSortMax (tile paths)
    const uint64_t cap = static_cast<uint64_t>(n) / (kSmallSort + 1) + 1;
    p->long_cap = static_cast<uint32_t>(cap < cells ? cap : cells);
    if (p->path == Path::kDirect) {
      p->off_long_count = off;
      off = align_up(off + 4u, 256);
      p->off_long = off;
      off = align_up(off + static_cast<size_t>(p->long_cap) * 4u, 256);
      if (p->move) {  // the scatter kernel's records, in arrival order
        p->off_unstable = off;
        off = align_up(off + static_cast<size_t>(n) * 32u, 256);
      }
    } else {  // FixLists: header, short list (one entry per cell of two or more), long list,
              // arrival-order indices of the tiles with a long cell (n words)
      const uint64_t fcap = static_cast<uint64_t>(n) / 2 + 1;
      p->fix_cap = static_cast<uint32_t>(fcap < cells ? fcap : cells);
      p->off_fix = off;
      off = align_up(off + (static_cast<size_t>(kFixHeader) + p->fix_cap + p->long_cap + n) * 4u, 256);
    }
  }
  p->total = off ? off : 256;
  return UGP_OK;
}

const char* stage_name(const Plan& p, uint32_t stage) {
  static const char* const kBucket[UGP_NUM_STAGES] = {"coarse_sort", "tile_scan", "rebucket", "tile_sort",
                                                     "stable_sort", "gather"};
  static const char* const kDirect[UGP_NUM_STAGES] = {"clear", "count", "scan", "scatter",
                                                      "stable_sort", "gather"};
  static const char* const kStaged[UGP_NUM_STAGES] = {"chunk_sort", nullptr, nullptr, "tile_sort",
                                                      "stable_sort", "gather"};
  static const char* const kSingleNames[UGP_NUM_STAGES] = {nullptr, nullptr, nullptr, "tile_sort",
                                                           "stable_sort", "gather"};
  if (stage >= UGP_NUM_STAGES) return nullptr;
  if (p.path == Path::kEmpty) return stage == 0 ? "clear" : nullptr;
  if (p.path == Path::kStaged && stage < 4) return kStaged[stage];
  if (p.path == Path::kSingle && stage < 4) return kSingleNames[stage];
  if (stage == 4 && !p.stable) return nullptr;
  if (stage == 5 && !p.gather) return nullptr;
  return p.path == Path::kBucketed ? kBucket[stage] : kDirect[stage];
}

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(const Span& a, const Span& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

Span span_of(const void* ptr, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
  return Span{lo, lo + bytes};
}

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
  uint32_t capacity;  // overflow diagnostics: capacity per cell
  uint32_t* diag;     // overflow diagnostics out (2 words), or nullptr
};

int validate(const BuildArgs& a, Plan* plan) {
  if (!a.origin || !a.dims) return UGP_ERR_NULL;
  int st = make_plan(a.n, a.dims, a.flags, plan);
  if (st != UGP_OK) return st;
  // a usable cell size is any finite positive float (subnormal ones too:
  // the kernels keep fp32 subnormals and divide correctly rounded)
  if (!std::isfinite(a.cell_size) || !(a.cell_size > 0.0f)) return UGP_ERR_ARG;
  for (int k = 0; k < 3; ++k)
    if (!std::isfinite(a.origin[k])) return UGP_ERR_ARG;
  if (!a.conteos || !a.inicios || !a.workspace) return UGP_ERR_NULL;
  const bool writes_records = (a.flags & UGP_FLAG_INDEX_ONLY) == 0;
  if (a.n > 0 && (!a.particles || !a.celdaDe || !a.ordenado || (writes_records && !a.reordered)))
    return UGP_ERR_NULL;
  if (!aligned(a.conteos, 16) || !aligned(a.inicios, 16) || !aligned(a.workspace, 256))
    return UGP_ERR_ALIGN;
  if (a.n > 0 && (!aligned(a.particles, 16) || (writes_records && !aligned(a.reordered, 16)) ||
                  !aligned(a.celdaDe, 16) || !aligned(a.ordenado, 16)))
    return UGP_ERR_ALIGN;
  if (a.diag && !aligned(a.diag, 4)) return UGP_ERR_ALIGN;
  if (a.workspace_bytes < plan->total) return UGP_ERR_WORKSPACE;
  const size_t n = a.n;
  const size_t c = plan->cells;
  const Span spans[8] = {
      span_of(a.particles, 32 * n),    span_of(a.celdaDe, 4 * n),   span_of(a.conteos, 4 * c),
      span_of(a.inicios, 4 * (c + 1)), span_of(a.ordenado, 4 * n),
      span_of(a.reordered, writes_records ? 32 * n : 0),
      span_of(a.workspace, plan->total), span_of(a.diag, a.diag ? 8 : 0),
  };
  for (int i = 0; i < 8; ++i)
    for (int j = i + 1; j < 8; ++j)
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
  g.morton = (a.flags & UGP_FLAG_MORTON) ? 1u : 0u;
  return g;
}

void launch_clear(uint32_t* ptr, uint64_t words, uint32_t* extra, uint32_t extra_words,
                  hipStream_t s) {
  const uint64_t vec = words / 4;
  uint32_t blocks = blocks_for(vec ? vec : 1, kBlock);
  if (blocks > 2048) blocks = 2048;
  launch(clear_kernel, dim3(blocks), dim3(kBlock), 0, s, ptr, words, extra, extra_words);
}

// Overflow diagnostics of a final conteos array (the direct path, and the
// standalone entry point): one launch whose last workgroup writes both
// words, with per-workgroup partials in one slot of diag_scratch. Slots are
// dealt round robin, so up to kDiagSlots launches may be in flight at once
// on one GPU (more race on a slot).
int enqueue_cell_diag(const uint32_t* conteos, uint64_t cells, uint32_t cap, uint32_t* diag,
                      hipStream_t s) {
  void* base = nullptr;
  const int st = symbol_address(HIP_SYMBOL(diag_scratch), g_diag_scratch_ptr, &base);
  if (st != UGP_OK) return st;
  DiagScratch* sc = static_cast<DiagScratch*>(base);
  const uint32_t slot = g_diag_slot.fetch_add(1u, std::memory_order_relaxed) % kDiagSlots;
  // two load rounds per workgroup: half as many workgroups take the ticket
  // one after another at the end, for the same bytes in flight
  uint32_t blocks = blocks_for((cells + 3) / 4, static_cast<uint64_t>(kDiagThreads) * kDiagItems * kDiagRounds);
  if (blocks > kDiagGrid) blocks = kDiagGrid;
  if (blocks == 0) blocks = 1;  // no cells: one workgroup writes the two zeros
  launch(cell_diag_kernel<kDiagThreads>, dim3(blocks), dim3(kDiagThreads), 0, s, conteos,
                     static_cast<uint32_t>(cells), cap, diag, &sc->ticket[slot], &sc->part[slot][0]);
  return UGP_OK;
}

// Where the scatter kernels write the records: nowhere (a gather follows, or
// index only), a workspace copy (stable mode on the direct path: the
// per-cell sort then writes `reordered`), or `reordered` itself.
uint4* record_dst(const BuildArgs& a, const Plan& p) {
  if (!p.move) return nullptr;
  if (p.stable && p.path == Path::kDirect)
    return reinterpret_cast<uint4*>(static_cast<char*>(a.workspace) + p.off_unstable);
  return reinterpret_cast<uint4*>(a.reordered);
}

// the shared scatter of the tile paths (no queue otherwise)
TileQueue tile_queue_of(const BuildArgs& a, const Plan& p) {
  TileQueue q{};
  if (!p.queue) return q;
  q.base = reinterpret_cast<uint32_t*>(static_cast<char*>(a.workspace) + p.off_queue);
  q.sources = reinterpret_cast<uint32_t*>(static_cast<char*>(a.workspace) + p.off_sources);
  q.slot_words = (1u << p.tile_shift) + kQueueRunWords;
  q.run_off = 1u << p.tile_shift;
  return q;
}

// the stable fix-up lists of the tile paths (null otherwise)
FixLists fix_lists_of(const BuildArgs& a, const Plan& p) {
  FixLists fl{};
  if (!p.stable || p.path == Path::kDirect) return fl;
  fl.base = reinterpret_cast<uint32_t*>(static_cast<char*>(a.workspace) + p.off_fix);
  fl.fix_cap = p.fix_cap;
  fl.long_cap = p.long_cap;
  return fl;
}

// The stable-order pass of every path, and the gather pass.
void enqueue_stable_sort(const BuildArgs& a, const Plan& p, char* ws) {
  const uint4* parts = reinterpret_cast<const uint4*>(a.particles);
  uint4* out = p.move ? reinterpret_cast<uint4*>(a.reordered) : nullptr;
  if (p.path != Path::kDirect) {
    // the tile kernel put every cell it could in order and listed the rest
    // (list lengths zeroed by the build's first kernel): one pass over them,
    // records read from the input by particle index
    const FixLists fl = fix_lists_of(a, p);
    const uint32_t long_blocks = (p.long_cap < kFixLongBlocks) ? p.long_cap : kFixLongBlocks;
    const uint32_t short_blocks = blocks_for(p.fix_cap, kSortBlock);  // 64 entries per wave
    const dim3 grid(long_blocks + ((short_blocks < kFixShortBlocks) ? short_blocks : kFixShortBlocks));
    if (p.move)
      launch(fix_cells_kernel<true>, grid, dim3(kSortBlock), 0, a.stream, a.inicios, a.celdaDe,
                         static_cast<uint32_t>(p.cells), a.n, fl, long_blocks, a.ordenado, parts, out);
    else
      launch(fix_cells_kernel<false>, grid, dim3(kSortBlock), 0, a.stream, a.inicios, a.celdaDe,
                         static_cast<uint32_t>(p.cells), a.n, fl, long_blocks, a.ordenado, nullptr, nullptr);
    return;
  }
  uint32_t* long_count = reinterpret_cast<uint32_t*>(ws + p.off_long_count);
  uint32_t* long_list = reinterpret_cast<uint32_t*>(ws + p.off_long);
  const uint32_t cells = static_cast<uint32_t>(p.cells);
  launch_clear(long_count, 1, nullptr, 0, a.stream);
  const dim3 grid(blocks_for(cells, kBlock));
  if (p.move) {
    launch(sort_short_cells_kernel<true>, grid, dim3(kBlock), 0, a.stream, a.inicios, cells, a.n,
                       a.ordenado, long_list, p.long_cap, long_count,
                       reinterpret_cast<const uint4*>(ws + p.off_unstable), out);
    launch(sort_long_cells_kernel<true>, dim3(kSortGrid), dim3(kSortBlock), 0, a.stream,
                       a.inicios, a.celdaDe, a.n, long_list, p.long_cap, long_count, a.ordenado, parts, out);
  } else {
    launch(sort_short_cells_kernel<false>, grid, dim3(kBlock), 0, a.stream, a.inicios, cells, a.n,
                       a.ordenado, long_list, p.long_cap, long_count, nullptr, nullptr);
    launch(sort_long_cells_kernel<false>, dim3(kSortGrid), dim3(kSortBlock), 0, a.stream,
                       a.inicios, a.celdaDe, a.n, long_list, p.long_cap, long_count, a.ordenado, nullptr,
                       nullptr);
  }
}

void enqueue_gather(const BuildArgs& a) {
  launch(gather_kernel, dim3(blocks_for(a.n, kBlock * kGatherItems / 2)), dim3(kBlock),
                     0, a.stream, a.ordenado, a.n, a.n, reinterpret_cast<const uint4*>(a.particles),
                     reinterpret_cast<uint4*>(a.reordered));
}

// the staged tile kernel over tiles given by rows (staged: chunk rows;
// bucketed: one contiguous run per tile; SINGLE: the one tile over the
// input, no rows), with or without records, diagnostics and stable order
template <bool SINGLE>
void launch_tile_sort(const BuildArgs& a, const Plan& p, const uint2* rows, const uint4* rec,
                      const uint32_t* idx) {
  const uint32_t cells = static_cast<uint32_t>(p.cells);
  uint4* dst = record_dst(a, p);
  const dim3 grid(p.ntiles);
  hipStream_t s = a.stream;
  const FixLists fl = fix_lists_of(a, p);
  const GridParams g = grid_params(a);
  uint32_t* keys_out = SINGLE ? a.celdaDe : nullptr;
  const TileQueue q = SINGLE ? TileQueue{} : tile_queue_of(a, p);
  const uint32_t packed = (p.path == Path::kStaged) ? 1u : 0u;  // chunk_sort's index words
  // one instantiation per (moves records, diagnostics, stable order)
#define UGP_TILE_SORT(M, D, S)                                                                        \
  launch_staged_cells<M, D, S, SINGLE>(p.tile_shift, grid, s, rows, p.nchunks, p.chunk, p.ntiles, g, \
                                       cells, a.n, rec, idx, a.conteos, a.inicios, a.ordenado, dst,  \
                                       D ? a.capacity : 0u, D ? a.diag : nullptr, fl, keys_out, q,   \
                                       packed)
  const bool m = p.move, d = a.diag != nullptr, st = p.stable;
  if (m && d && st) UGP_TILE_SORT(true, true, true);
  else if (m && d) UGP_TILE_SORT(true, true, false);
  else if (m && st) UGP_TILE_SORT(true, false, true);
  else if (m) UGP_TILE_SORT(true, false, false);
  else if (d && st) UGP_TILE_SORT(false, true, true);
  else if (d) UGP_TILE_SORT(false, true, false);
  else if (st) UGP_TILE_SORT(false, false, true);
  else UGP_TILE_SORT(false, false, false);
#undef UGP_TILE_SORT
}

// single tile: the tile kernel reads the input directly (one run, identity
// indices) and writes celdaDe itself
void enqueue_single(uint32_t stage, const BuildArgs& a, const Plan& p) {
  switch (stage) {
    case 3: {
      // without diagnostics or stable order (whose words one workgroup zeroes
      // for itself) the cells are split into up to 64 tiles (of at least 16
      // cells), each workgroup reading the whole input: many CUs on a
      // latency-bound build
      Plan q = p;
      if (!p.stable && a.diag == nullptr) {
        const uint32_t lg = p.tile_shift;  // the one tile covers 2^lg >= K keys
        q.tile_shift = (lg > kStagedMinShift + kSingleSplitLog) ? lg - kSingleSplitLog : kStagedMinShift;
        q.ntiles = static_cast<uint32_t>((p.cells + (1ull << q.tile_shift) - 1) >> q.tile_shift);
      }
      launch_tile_sort<true>(a, q, nullptr, reinterpret_cast<const uint4*>(a.particles), nullptr);
      break;
    }
    case 4:
      if (p.stable) enqueue_stable_sort(a, p, static_cast<char*>(a.workspace));
      break;
    case 5:
      if (p.gather) enqueue_gather(a);
      break;
    default:
      break;
  }
}

void enqueue_staged(uint32_t stage, const BuildArgs& a, const Plan& p) {
  char* ws = static_cast<char*>(a.workspace);
  uint2* rows = reinterpret_cast<uint2*>(ws + p.off_rows);
  uint4* chunk_rec = reinterpret_cast<uint4*>(ws + p.off_chunk_rec);
  uint32_t* chunk_idx = reinterpret_cast<uint32_t*>(ws + p.off_chunk_idx);
  hipStream_t s = a.stream;
  switch (stage) {
    case 0:
      if (p.chunk == kSmallChunk)
        launch(staged_keys_kernel<kSmallChunkThreads>, dim3(p.nchunks), dim3(kSmallChunkThreads), 0,
                           s, reinterpret_cast<const uint4*>(a.particles), a.n, grid_params(a), a.celdaDe, rows,
                           p.tile_shift, p.ntiles, chunk_rec, chunk_idx, a.diag, fix_lists_of(a, p).base,
                           tile_queue_of(a, p).base, 0u);
      else
        launch(staged_keys_kernel<kChunkThreads>, dim3(p.nchunks), dim3(kChunkThreads), 0, s,
                           reinterpret_cast<const uint4*>(a.particles), a.n, grid_params(a), a.celdaDe, rows,
                           p.tile_shift, p.ntiles, chunk_rec, chunk_idx, a.diag, fix_lists_of(a, p).base,
                           tile_queue_of(a, p).base, 0u);
      break;
    case 3:
      launch_tile_sort<false>(a, p, rows, chunk_rec, chunk_idx);
      break;
    case 4:
      if (p.stable) enqueue_stable_sort(a, p, ws);
      break;
    case 5:
      if (p.gather) enqueue_gather(a);
      break;
    default:
      break;
  }
}

void enqueue_bucketed(uint32_t stage, const BuildArgs& a, const Plan& p) {
  char* ws = static_cast<char*>(a.workspace);
  uint2* rows1 = reinterpret_cast<uint2*>(ws + p.off_rows1);
  uint4* coarse_rec = reinterpret_cast<uint4*>(ws + p.off_coarse_rec);
  uint32_t* coarse_idx = reinterpret_cast<uint32_t*>(ws + p.off_coarse_idx);
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws + p.off_hist);
  uint32_t* tile_total = reinterpret_cast<uint32_t*>(ws + p.off_tile_total);
  uint32_t* group_total = reinterpret_cast<uint32_t*>(ws + p.off_group_total);
  uint2* rows = reinterpret_cast<uint2*>(ws + p.off_rows);
  uint4* tile_rec = reinterpret_cast<uint4*>(ws + p.off_chunk_rec);
  uint32_t* tile_idx = reinterpret_cast<uint32_t*>(ws + p.off_chunk_idx);
  const uint32_t fpb = 1u << (p.cshift - p.tile_shift);
  hipStream_t s = a.stream;
  switch (stage) {
    case 0:  // chunks sorted by bucket: the chunk kernel with buckets for tiles
      launch(staged_keys_kernel<kChunkThreads>, dim3(p.ncoarse), dim3(kChunkThreads), 0, s,
             reinterpret_cast<const uint4*>(a.particles), a.n, grid_params(a), a.celdaDe, rows1, p.cshift,
             p.nbuckets, coarse_rec, coarse_idx, a.diag, fix_lists_of(a, p).base, tile_queue_of(a, p).base, 1u);
      break;
    case 1:
      launch(bucket_fine_count_kernel, dim3(p.ncount), dim3(kCountThreads), 0, s, a.celdaDe, a.n, p.tile_shift,
             p.ntiles, hist);
      launch(bucket_colscan_kernel, dim3(blocks_for(p.ntiles, 64)), dim3(kScanWaves * 64), 0, s, hist, p.ncount,
             p.ntiles, tile_total, group_total);
      break;
    case 2:
      launch(bucket_rebucket_kernel, dim3(p.nrb * p.nbuckets), dim3(kRbThreads), 0, s, rows1, p.ncoarse,
             p.nbuckets, coarse_rec, coarse_idx, p.nrb, p.tile_shift, fpb, p.ntiles, hist, tile_total, group_total,
             a.n, tile_rec, tile_idx, rows);
      break;
    case 3:
      launch_tile_sort<false>(a, p, rows, tile_rec, tile_idx);
      break;
    case 4:
      if (p.stable) enqueue_stable_sort(a, p, ws);
      break;
    case 5:
      if (p.gather) enqueue_gather(a);
      break;
    default:
      break;
  }
}

int enqueue_direct(uint32_t stage, const BuildArgs& a, const Plan& p) {
  char* ws = static_cast<char*>(a.workspace);
  uint32_t* cursor = reinterpret_cast<uint32_t*>(ws + p.off_cursor);
  uint32_t* tilesum = reinterpret_cast<uint32_t*>(ws + p.off_small);
  const uint32_t cells = static_cast<uint32_t>(p.cells);
  hipStream_t s = a.stream;
  const dim3 pgrid(blocks_for(a.n, kBlock * kCountItems));
  switch (stage) {
    case 0:
      launch_clear(a.conteos, p.cells, tilesum, p.nbins + kCounterWords, s);
      break;
    case 1:
      launch(count_kernel, pgrid, dim3(kBlock), 0, s,
                         reinterpret_cast<const float4*>(a.particles), a.n, grid_params(a),
                         a.celdaDe, a.conteos, tilesum, p.bin_shift, p.nbins);
      break;
    case 2:
      launch(scan_kernel, dim3(p.nbins), dim3(kBlock), 0, s, a.conteos, p.cells,
                         tilesum, p.bin_shift, a.inicios, cursor);
      break;
    case 3:
      if (!p.move)
        launch(scatter_kernel<false>, pgrid, dim3(kBlock), 0, s, a.celdaDe, a.n, cells,
                           cursor, a.ordenado, nullptr, nullptr);
      else
        launch(scatter_kernel<true>, pgrid, dim3(kBlock), 0, s, a.celdaDe, a.n, cells,
                           cursor, a.ordenado, reinterpret_cast<const uint4*>(a.particles),
                           record_dst(a, p));
      if (a.diag) {
        const int st = enqueue_cell_diag(a.conteos, p.cells, a.capacity, a.diag, s);
        if (st != UGP_OK) return st;
      }
      break;
    case 4:
      if (p.stable) enqueue_stable_sort(a, p, ws);
      break;
    case 5:
      if (p.gather) enqueue_gather(a);
      break;
    default:
      break;
  }
  return UGP_OK;
}

int enqueue_stage(uint32_t stage, const BuildArgs& a, const Plan& p) {
  if (stage >= UGP_NUM_STAGES) return UGP_ERR_ARG;
  switch (p.path) {
    case Path::kEmpty:
      if (stage == 0) {
        launch_clear(a.conteos, p.cells, a.diag, a.diag ? 2u : 0u, a.stream);
        launch_clear(a.inicios, p.cells + 1, nullptr, 0, a.stream);
      }
      break;
    case Path::kSingle:
      enqueue_single(stage, a, p);
      break;
    case Path::kStaged:
      enqueue_staged(stage, a, p);
      break;
    case Path::kBucketed:
      enqueue_bucketed(stage, a, p);
      break;
    case Path::kDirect: {
      const int st = enqueue_direct(stage, a, p);
      if (st != UGP_OK) return st;
      break;
    }
  }
  return hipGetLastError() == hipSuccess ? UGP_OK : UGP_ERR_HIP;
}

// Whether a stage slot of this plan is exactly one kernel launch (its
// timing can then be the kernel's own start and end).
bool single_kernel_stage(const Plan& p, uint32_t stage, bool diag) {
  switch (p.path) {
    case Path::kEmpty:
      return false;
    case Path::kSingle:
      return stage == 3 || (stage == 4 && p.stable) || (stage == 5 && p.gather);
    case Path::kStaged:
      return stage == 0 || stage == 3 || (stage == 4 && p.stable) || (stage == 5 && p.gather);
    case Path::kBucketed:  // slot 1 holds two kernels (count, column scan)
      return stage == 0 || stage == 2 || stage == 3 || (stage == 4 && p.stable) || (stage == 5 && p.gather);
    case Path::kDirect:
      return stage <= 2 || (stage == 3 && !diag) || (stage == 5 && p.gather);
  }
  return false;
}

BuildArgs make_args(const ugp_particle* particles, uint32_t n, const float origin[3],
                    float cell_size, const uint32_t dims[3], uint32_t* celdaDe, uint32_t* conteos,
                    uint32_t* inicios, uint32_t* ordenado, ugp_particle* reordered, void* workspace,
                    size_t workspace_bytes, uint32_t flags, void* stream) {
  return BuildArgs{particles, n,        origin,          cell_size, dims,
                   celdaDe,   conteos,  inicios,         ordenado,  reordered,
                   workspace, workspace_bytes, flags, static_cast<hipStream_t>(stream),
                   0u,        nullptr};
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
    case UGP_ERR_ARG: return "invalid argument (cell_size, origin, flags, stage or events)";
    case UGP_ERR_RANGE: return "grid dimensions out of range (each dim in [1, 2^24], cells <= 2^32-2)";
    case UGP_ERR_ALIAS: return "two buffers overlap";
    case UGP_ERR_ALIGN: return "misaligned buffer (arrays need 16-byte, workspace 256-byte alignment)";
    case UGP_ERR_WORKSPACE: return "workspace too small";
    case UGP_ERR_HIP: return "HIP runtime error while enqueueing";
    default: return "unknown status";
  }
}

int ugp_grid_key_count(const uint32_t dims[3], uint32_t flags, uint64_t* keys) {
  if (!keys) return UGP_ERR_NULL;
  Plan p;
  const int st = make_plan(0, dims, flags, &p);
  if (st != UGP_OK) return st;
  *keys = p.cells;
  return UGP_OK;
}

int ugp_grid_workspace_bytes(uint32_t n, const uint32_t dims[3], uint32_t flags, size_t* bytes) {
  if (!bytes) return UGP_ERR_NULL;
  Plan p;
  const int st = make_plan(n, dims, flags, &p);
  if (st != UGP_OK) return st;
  *bytes = p.total;
  return UGP_OK;
}

const char* ugp_grid_stage_name(uint32_t n, const uint32_t dims[3], uint32_t flags,
                                uint32_t stage) {
  Plan p;
  if (make_plan(n, dims, flags, &p) != UGP_OK) return nullptr;
  return stage_name(p, stage);
}

int ugp_grid_build_stage(uint32_t stage, const ugp_particle* particles, uint32_t n,
                         const float origin[3], float cell_size, const uint32_t dims[3],
                         uint32_t* celdaDe, uint32_t* conteos, uint32_t* inicios,
                         uint32_t* ordenado, ugp_particle* reordered, void* workspace,
                         size_t workspace_bytes, uint32_t flags, void* stream) {
  if (stage >= UGP_NUM_STAGES) return UGP_ERR_ARG;
  const BuildArgs a = make_args(particles, n, origin, cell_size, dims, celdaDe, conteos, inicios,
                                ordenado, reordered, workspace, workspace_bytes, flags, stream);
  Plan p;
  const int st = validate(a, &p);
  if (st != UGP_OK) return st;
  return enqueue_stage(stage, a, p);
}

int ugp_grid_build(const ugp_particle* particles, uint32_t n, const float origin[3],
                   float cell_size, const uint32_t dims[3], uint32_t* celdaDe, uint32_t* conteos,
                   uint32_t* inicios, uint32_t* ordenado, ugp_particle* reordered, void* workspace,
                   size_t workspace_bytes, uint32_t flags, void* stream) {
  const BuildArgs a = make_args(particles, n, origin, cell_size, dims, celdaDe, conteos, inicios,
                                ordenado, reordered, workspace, workspace_bytes, flags, stream);
  Plan p;
  int st = validate(a, &p);
  if (st != UGP_OK) return st;
  for (uint32_t stage = 0; stage < UGP_NUM_STAGES; ++stage) {
    st = enqueue_stage(stage, a, p);
    if (st != UGP_OK) return st;
  }
  return UGP_OK;
}

int ugp_grid_build_noalloc(const ugp_particle* particles, uint32_t n, const float origin[3],
                           float cell_size, const uint32_t dims[3], uint32_t* celdaDe, uint32_t* conteos,
                           uint32_t* inicios, uint32_t* ordenado, ugp_particle* reordered, uint32_t flags,
                           void* stream) {
  Plan p;
  if (!dims) return UGP_ERR_NULL;
  int st = make_plan(n, dims, flags, &p);
  if (st != UGP_OK) return st;
  if (p.total > UGP_NOALLOC_SCRATCH_BYTES) return UGP_ERR_WORKSPACE;
  void* ws = nullptr;
  st = symbol_address(HIP_SYMBOL(scratch), g_scratch_ptr, &ws);
  if (st != UGP_OK) return st;
  const BuildArgs a = make_args(particles, n, origin, cell_size, dims, celdaDe, conteos, inicios, ordenado,
                                reordered, ws, UGP_NOALLOC_SCRATCH_BYTES, flags, stream);
  st = validate(a, &p);
  if (st != UGP_OK) return st;
  for (uint32_t stage = 0; stage < UGP_NUM_STAGES; ++stage) {
    st = enqueue_stage(stage, a, p);
    if (st != UGP_OK) return st;
  }
  return UGP_OK;
}

int ugp_grid_build_diag(const ugp_particle* particles, uint32_t n, const float origin[3],
                        float cell_size, const uint32_t dims[3], uint32_t* celdaDe,
                        uint32_t* conteos, uint32_t* inicios, uint32_t* ordenado,
                        ugp_particle* reordered, void* workspace, size_t workspace_bytes,
                        uint32_t capacity, uint32_t* diag, uint32_t flags, void* stream) {
  if (!diag) return UGP_ERR_NULL;
  BuildArgs a = make_args(particles, n, origin, cell_size, dims, celdaDe, conteos, inicios,
                          ordenado, reordered, workspace, workspace_bytes, flags, stream);
  a.capacity = capacity;
  a.diag = diag;
  Plan p;
  int st = validate(a, &p);
  if (st != UGP_OK) return st;
  for (uint32_t stage = 0; stage < UGP_NUM_STAGES; ++stage) {
    st = enqueue_stage(stage, a, p);
    if (st != UGP_OK) return st;
  }
  return UGP_OK;
}

int ugp_cell_diag(const uint32_t* conteos, uint32_t cells, uint32_t capacity, uint32_t* diag,
                  void* stream) {
  if (!diag || (cells > 0 && !conteos)) return UGP_ERR_NULL;
  if (!aligned(diag, 4) || (cells > 0 && !aligned(conteos, 16))) return UGP_ERR_ALIGN;
  if (overlap(span_of(conteos, 4ull * cells), span_of(diag, 8))) return UGP_ERR_ALIAS;
  const int st = enqueue_cell_diag(conteos, cells, capacity, diag, static_cast<hipStream_t>(stream));
  if (st != UGP_OK) return st;
  return hipGetLastError() == hipSuccess ? UGP_OK : UGP_ERR_HIP;
}

int ugp_cell_diag_timed(const uint32_t* conteos, uint32_t cells, uint32_t capacity, uint32_t* diag,
                        void* stream, void* event_before, void* event_after) {
  if (!event_before || !event_after) return UGP_ERR_ARG;
  g_timed_launch = TimedLaunch{static_cast<hipEvent_t>(event_before), static_cast<hipEvent_t>(event_after)};
  const int st = ugp_cell_diag(conteos, cells, capacity, diag, stream);
  g_timed_launch = TimedLaunch{};  // disarmed also when the call failed before its launch
  return st;
}

int ugp_neighbor_count(const ugp_particle* particles, uint32_t n, const float origin[3],
                       float cell_size, const uint32_t dims[3], const uint32_t* inicios,
                       const uint32_t* ordenado, float radius, uint32_t* counts, uint32_t flags,
                       void* stream) {
  if (!origin || !dims) return UGP_ERR_NULL;
  if (flags & ~UGP_FLAG_MORTON) return UGP_ERR_ARG;
  Plan p;
  int st = make_plan(n, dims, flags, &p);
  if (st != UGP_OK) return st;
  if (!std::isfinite(cell_size) || !(cell_size > 0.0f)) return UGP_ERR_ARG;
  for (int k = 0; k < 3; ++k)
    if (!std::isfinite(origin[k])) return UGP_ERR_ARG;
  if (!std::isfinite(radius) || !(radius >= 0.0f)) return UGP_ERR_ARG;
  if (n == 0) return UGP_OK;
  if (!particles || !inicios || !counts) return UGP_ERR_NULL;
  if (!aligned(particles, 16) || !aligned(inicios, 4) || !aligned(counts, 4) ||
      (ordenado && !aligned(ordenado, 4)))
    return UGP_ERR_ALIGN;
  const Span sc = span_of(counts, 4ull * n);
  if (overlap(sc, span_of(particles, 32ull * n)) || overlap(sc, span_of(inicios, 4 * (p.cells + 1))) ||
      overlap(sc, span_of(ordenado, ordenado ? 4ull * n : 0)))
    return UGP_ERR_ALIAS;
  BuildArgs a = make_args(particles, n, origin, cell_size, dims, nullptr, nullptr, nullptr, nullptr,
                          nullptr, nullptr, 0, flags, stream);
  const GridParams g = grid_params(a);
  const float r2 = radius * radius;
  const dim3 grid(blocks_for(n, kNeighborBlock)), block(kNeighborBlock);
  const float4* pf = reinterpret_cast<const float4*>(particles);
  hipStream_t s = a.stream;
  const bool morton = (flags & UGP_FLAG_MORTON) != 0;
  if (ordenado && morton)
    launch((neighbor_count_kernel<true, true>), grid, block, 0, s, pf, n, g, dims[1], dims[2],
                       inicios, ordenado, r2, counts);
  else if (ordenado)
    launch((neighbor_count_kernel<true, false>), grid, block, 0, s, pf, n, g, dims[1], dims[2],
                       inicios, ordenado, r2, counts);
  else if (morton)
    launch((neighbor_count_kernel<false, true>), grid, block, 0, s, pf, n, g, dims[1], dims[2],
                       inicios, nullptr, r2, counts);
  else
    launch((neighbor_count_kernel<false, false>), grid, block, 0, s, pf, n, g, dims[1], dims[2],
                       inicios, nullptr, r2, counts);
  return hipGetLastError() == hipSuccess ? UGP_OK : UGP_ERR_HIP;
}

int ugp_grid_build_timed(const ugp_particle* particles, uint32_t n, const float origin[3],
                         float cell_size, const uint32_t dims[3], uint32_t* celdaDe,
                         uint32_t* conteos, uint32_t* inicios, uint32_t* ordenado,
                         ugp_particle* reordered, void* workspace, size_t workspace_bytes,
                         uint32_t flags, void* stream, uint32_t timed_stage, void* event_before,
                         void* event_after) {
  if (timed_stage >= UGP_NUM_STAGES || !event_before || !event_after) return UGP_ERR_ARG;
  const BuildArgs a = make_args(particles, n, origin, cell_size, dims, celdaDe, conteos, inicios,
                                ordenado, reordered, workspace, workspace_bytes, flags, stream);
  Plan p;
  int st = validate(a, &p);
  if (st != UGP_OK) return st;
  hipEvent_t ev0 = static_cast<hipEvent_t>(event_before), ev1 = static_cast<hipEvent_t>(event_after);
  const bool one_kernel = single_kernel_stage(p, timed_stage, false);
  for (uint32_t stage = 0; stage < UGP_NUM_STAGES; ++stage) {
    const bool timed = stage == timed_stage;
    if (timed) {
      if (one_kernel) {
        g_timed_launch = TimedLaunch{ev0, ev1};  // the stage's kernel records them itself
      } else if (hipEventRecord(ev0, a.stream) != hipSuccess) {
        return UGP_ERR_HIP;
      }
    }
    st = enqueue_stage(stage, a, p);
    if (timed && one_kernel && g_timed_launch.start != nullptr) {
      // no kernel took the events (a stage that enqueued nothing): record an empty interval
      g_timed_launch = TimedLaunch{};
      if (st == UGP_OK && (hipEventRecord(ev0, a.stream) != hipSuccess || hipEventRecord(ev1, a.stream) != hipSuccess))
        return UGP_ERR_HIP;
    }
    if (st != UGP_OK) return st;
    if (timed && !one_kernel && hipEventRecord(ev1, a.stream) != hipSuccess) return UGP_ERR_HIP;
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
  const Span si = span_of(in, 4ull * count);
  const Span so = span_of(out, 4ull * (count + 1ull));
  const Span sw = span_of(workspace, need);
  if (overlap(si, so) || overlap(si, sw) || overlap(so, sw)) return UGP_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* tilesum = static_cast<uint32_t*>(workspace);
  if (count == 0) {
    launch_clear(out, 1, nullptr, 0, s);  // out[0] = 0
    return hipGetLastError() == hipSuccess ? UGP_OK : UGP_ERR_HIP;
  }
  const uint32_t lg = ceil_log2_u64(count);
  const uint32_t shift = (lg > kMinBinShift + 9) ? lg - 9 : kMinBinShift;
  const uint32_t nbins =
      static_cast<uint32_t>((static_cast<uint64_t>(count) + (1ull << shift) - 1) >> shift);
  launch(tile_reduce_kernel, dim3(nbins), dim3(kBlock), 0, s, in,
                     static_cast<uint64_t>(count), shift, tilesum);
  launch(scan_kernel, dim3(nbins), dim3(kBlock), 0, s, in, static_cast<uint64_t>(count),
                     tilesum, shift, out, nullptr);
  return hipGetLastError() == hipSuccess ? UGP_OK : UGP_ERR_HIP;
}

int ugp_reorder_arrays(const uint32_t* idx, uint32_t n, uint32_t n_src, const ugp_array_desc* arrays,
                       uint32_t count, void* stream) {
  if (count == 0 || count > kMaxArrays) return UGP_ERR_ARG;
  if (!arrays) return UGP_ERR_NULL;
  uint32_t bytes = 0;
  bool vec16 = true;
  for (uint32_t q = 0; q < count; ++q) {
    const ugp_array_desc& d = arrays[q];
    // an element's 4-byte chunks must fit one workgroup; checked per array
    // first so that the sum below cannot wrap
    if (d.elem_bytes == 0 || d.elem_bytes % 4 != 0 || d.elem_bytes / 4u > static_cast<uint32_t>(kBlock))
      return UGP_ERR_ARG;
    bytes += d.elem_bytes;
    if (n > 0 && (!d.src || !d.dst)) return UGP_ERR_NULL;
    if (!aligned(d.src, 4) || !aligned(d.dst, 4)) return UGP_ERR_ALIGN;
    vec16 = vec16 && d.elem_bytes % 16 == 0 && aligned(d.src, 16) && aligned(d.dst, 16);
  }
  const uint32_t chunk = vec16 ? 16u : 4u;
  if (bytes / chunk > static_cast<uint32_t>(kBlock)) return UGP_ERR_ARG;  // one element's chunks fit a workgroup
  if (n == 0) return UGP_OK;
  if (!idx) return UGP_ERR_NULL;
  if (!aligned(idx, 4)) return UGP_ERR_ALIGN;
  // no destination may overlap the index, a source, or another destination
  const Span si = span_of(idx, 4ull * n);
  for (uint32_t q = 0; q < count; ++q) {
    const Span dq = span_of(arrays[q].dst, static_cast<size_t>(arrays[q].elem_bytes) * n);
    if (overlap(dq, si)) return UGP_ERR_ALIAS;
    for (uint32_t r = 0; r < count; ++r) {
      if (overlap(dq, span_of(arrays[r].src, static_cast<size_t>(arrays[r].elem_bytes) * n_src)))
        return UGP_ERR_ALIAS;
      if (r != q && overlap(dq, span_of(arrays[r].dst, static_cast<size_t>(arrays[r].elem_bytes) * n)))
        return UGP_ERR_ALIAS;
    }
  }
  if (n_src == 0) return UGP_OK;  // every index is out of range: nothing to write
  ArraySet set{};
  set.count = count;
  set.first[0] = 0;
  for (uint32_t q = 0; q < count; ++q) {
    set.src[q] = arrays[q].src;
    set.dst[q] = arrays[q].dst;
    set.chunks[q] = arrays[q].elem_bytes / chunk;
    set.first[q + 1] = set.first[q] + set.chunks[q];
  }
  const uint32_t per = kBlock / set.first[count];
  const dim3 grid(blocks_for(n, static_cast<uint64_t>(per) * kArrayItems));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (vec16)
    launch(gather_arrays_kernel<uint4>, grid, dim3(kBlock), 0, s, idx, n, n_src, set);
  else
    launch(gather_arrays_kernel<uint32_t>, grid, dim3(kBlock), 0, s, idx, n, n_src, set);
  return hipGetLastError() == hipSuccess ? UGP_OK : UGP_ERR_HIP;
}

int ugp_reorder(const ugp_particle* src, uint32_t n_src, const uint32_t* idx, uint32_t n,
                ugp_particle* dst, void* stream) {
  if (n == 0) return UGP_OK;
  if (!src || !idx || !dst) return UGP_ERR_NULL;
  if (!aligned(src, 16) || !aligned(dst, 16) || !aligned(idx, 4)) return UGP_ERR_ALIGN;
  const Span ss = span_of(src, 32ull * n_src);
  const Span si = span_of(idx, 4ull * n);
  const Span sd = span_of(dst, 32ull * n);
  if (overlap(ss, sd) || overlap(si, sd)) return UGP_ERR_ALIAS;
  if (n_src == 0) return UGP_OK;  // every index is out of range: nothing to write
  launch(gather_kernel, dim3(blocks_for(n, kBlock * kGatherItems / 2)), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), idx, n, n_src,
                     reinterpret_cast<const uint4*>(src), reinterpret_cast<uint4*>(dst));
  return hipGetLastError() == hipSuccess ? UGP_OK : UGP_ERR_HIP;
}

}  // extern "C"
