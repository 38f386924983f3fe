/*
 * ugp.h -- C ABI of the uniform-grid particle index build for MI355X (gfx950).
 *
 * The build is a counting sort of particles by cell key, in the steps the
 * source pages describe:
 *
 *   1. count   -- every particle's cell index is stored per particle
 *                 (celdaDe) and counted into a per-cell histogram (conteos).
 *                 Page "Contar partículas por celda", section "El kernel".
 *   2. scan    -- the exclusive prefix sum of the histogram gives the first
 *                 slot of every cell (inicios), with one extra trailing slot
 *                 holding the total, so cell c is [inicios[c], inicios[c+1]).
 *                 Page "Construir el índice de la rejilla con un prefix sum",
 *                 section "Del conteo al inicio".
 *   3. scatter -- a per-cell atomic cursor hands out slots inside each cell's
 *                 range and the particle index is written there (ordenado).
 *                 Same page, section "La dispersión".
 *   4. reorder -- the 32-byte records are copied into cell order in a second
 *                 buffer (reordered[k] = particles[ordenado[k]]).
 *                 Page "Reordenar por celda y la coalescencia de memoria",
 *                 section "El kernel de reordenación".
 *
 * Cell key (the pages name it but leave its body to an earlier lesson; this
 * is the reading the rest of the pages support): on each axis a,
 *     t = p[a] - origin[a]            (binary32 subtraction)
 *     q = t / cell_size               (correctly rounded binary32 division)
 *     k[a] = floor(q) clamped to [0, dims[a]-1]   (NaN and -inf -> 0, +inf -> dims[a]-1)
 * and celdaDe = k[0] + k[1]*dims[0] + k[2]*dims[0]*dims[1] (the linear order of
 * "Reordenar por celda...", section "El orden de las celdas también importa").
 * Points outside the domain, NaN and infinities are clamped, never errors.
 *
 * Conventions for every entry point below:
 *  - Device pointers are HIP device memory on the current device; host
 *    pointers are read before the call returns.
 *  - The caller allocates and owns every buffer. The library never
 *    allocates or frees memory and never synchronises the host with the
 *    device. It keeps no state between calls except two fixed device arrays
 *    of its own per GPU (zero at load): the per-workgroup partials of
 *    ugp_cell_diag() (left ready for the next launch by every launch), and
 *    the workspace of ugp_grid_build_noalloc().
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    The call returns once the work is enqueued; outputs are valid when the
 *    stream reaches that point, and inputs must not change before then.
 *  - Arguments are validated on the host before anything is enqueued; on
 *    any error nothing is enqueued and the status code says why. A launch
 *    failure reported by the HIP runtime returns UGP_ERR_HIP.
 *  - All u32 arrays and the particle arrays must be 16-byte aligned (any
 *    torch/hipMalloc allocation is); the workspace must be 256-byte aligned.
 *  - No two buffers passed to one call may overlap.
 */
#ifndef UGP_H
#define UGP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One particle: 32 bytes, fields at offsets 0 / 12 / 16 / 28.
 * Page "El estado de las partículas en storage buffers", section
 * "La estructura y su alineación". Records are copied bit for bit. */
typedef struct ugp_particle {
    float pos[3];
    float vida;
    float vel[3];
    float masa;
} ugp_particle;

/* Status codes. */
#define UGP_OK 0
#define UGP_ERR_NULL (-1)      /* a required pointer is NULL */
#define UGP_ERR_ARG (-2)       /* cell_size not a finite normal positive float, origin not finite, unknown flag, stage or event */
#define UGP_ERR_RANGE (-3)     /* a dim is 0 or > 2^24, or the cell count exceeds 2^32-2 */
#define UGP_ERR_ALIAS (-4)     /* two buffers overlap */
#define UGP_ERR_ALIGN (-5)     /* an array is not 16-byte aligned, or the workspace not 256-byte aligned */
#define UGP_ERR_WORKSPACE (-6) /* workspace smaller than ugp_grid_workspace_bytes() */
#define UGP_ERR_HIP (-7)       /* the HIP runtime reported an error while enqueueing */

/* Flags. */
/* Stable order: every cell lists its particle indices in ascending order,
 * the unique order a sequential counting sort gives (tie-break by particle
 * index, page "Construir el índice...", section "El orden dentro de la
 * celda"). Without it the order inside a cell depends on atomic arrival
 * order (same section): the grouping is exact, the order is not. */
#define UGP_FLAG_STABLE 0x1u
/* Reorder with a separate gather kernel (coalesced writes, scattered
 * reads) instead of writing the record inside the scatter kernel. The
 * result is identical; this only selects the kernel schedule. */
#define UGP_FLAG_GATHER 0x2u
/* Number cells along the Z (Morton) curve instead of x + y*nx + z*nx*ny
 * (page "Reordenar por celda y la coalescencia de memoria", section "El
 * orden de las celdas también importa"). The key of cell (x, y, z) puts bit
 * b of x, y, z at key bits 3b, 3b+1, 3b+2; every axis is padded to B bits,
 * 2^B being the smallest power of two >= the largest dimension, so there are
 * K = 2^(3B) keys (K = C on a cubic power-of-two grid; on other grids some
 * keys hold no cell and always count 0). Requires B <= 10 (UGP_ERR_RANGE
 * otherwise). celdaDe, conteos, inicios and the order of ordenado and
 * reordered are then in keys: conteos has K entries and inicios K+1
 * (ugp_grid_key_count()). */
#define UGP_FLAG_MORTON 0x4u
/* Build the index only: celdaDe, conteos, inicios and ordenado as usual,
 * `reordered` neither written nor required (may be NULL). For reordering
 * every few frames (page "Reordenar por celda...", section "Reordenar o
 * no"): between reorders the caller keeps its array, rebuilds the index of
 * the slightly moved particles, and reaches them through ordenado, which
 * then points to nearby positions. */
#define UGP_FLAG_INDEX_ONLY 0x8u

/* Pipeline stage slots, for ugp_grid_build_stage() / ugp_grid_build_timed().
 * The library picks one of five execution paths from n and the key count K
 * (ugp_grid_key_count(); the cell count C unless UGP_FLAG_MORTON);
 * each path fills the six slots with its own kernels, named by
 * ugp_grid_stage_name():
 *   n == 0            slot 0 "clear" (zero conteos and inicios); others empty
 *   n <= 8192 and K <= 2^14
 *                     -, -, -, "tile_sort" -- one launch: up to 64 workgroups
 *                     each read the whole input and build the index of their
 *                     own cells, celdaDe included
 *   K <= 2^22 and n <= 2^21 (K up to 2^23 on dense grids)
 *                     "chunk_sort", -, -, "tile_sort" -- two kernels, no
 *                     global atomics, records moved through LDS
 *   other K <= 2^26   "coarse_sort", "tile_scan", "rebucket", "tile_sort"
 *                     -- chunks sorted by bucket of 64 tiles, a per-tile
 *                     count and its column scan (two kernels), the
 *                     buckets' runs regrouped by tile, then the same tile
 *                     kernel; no global atomics, every record moved in runs
 *   larger K          "clear", "count", "scan", "scatter"     -- one global
 *                     atomic per particle in count and in scatter
 *   slot 4 "stable_sort" (UGP_FLAG_STABLE only; page "Construir el índice
 *   de la rejilla con un prefix sum", section "El orden dentro de la
 *   celda"). On the two tile paths the tile kernel already puts every cell
 *   of up to 256 particles in ascending particle index and lists the rest;
 *   this slot orders the listed cells: those of up to 256 in place (indices
 *   and records permuted inside the cell's slice), longer ones from a
 *   workspace copy of their arrival order, records gathered from the input.
 *   On the direct path it orders every cell's slice and writes the records
 *   in that order. Slot 5 "gather" (UGP_FLAG_GATHER only). */
#define UGP_NUM_STAGES 6u

/* Number of cell keys K for a grid and flags: C = dims[0]*dims[1]*dims[2]
 * for the linear numbering, 2^(3B) with UGP_FLAG_MORTON. conteos holds K
 * entries and inicios K+1. Writes *keys; returns UGP_OK, UGP_ERR_NULL,
 * UGP_ERR_RANGE or UGP_ERR_ARG. Pure host function. */
int ugp_grid_key_count(const uint32_t dims[3], uint32_t flags, uint64_t *keys);

/* Bytes of device workspace ugp_grid_build() needs for n particles on a
 * dims[0] x dims[1] x dims[2] grid with the given flags.
 * dims: host array of 3. Writes *bytes; returns UGP_OK or UGP_ERR_NULL /
 * UGP_ERR_RANGE / UGP_ERR_ARG. Pure host function. */
int ugp_grid_workspace_bytes(uint32_t n, const uint32_t dims[3], uint32_t flags, size_t *bytes);

/* Build the uniform-grid index of n particles.
 *
 *   particles   device, in:  n records (ugp_particle), read only
 *   n           number of particles (0 is valid: conteos and inicios are
 *               zeroed and nothing else is written)
 *   origin      host, in:    3 floats, lower corner of cell (0,0,0)
 *   cell_size   edge length of a cubic cell: finite and positive (a
 *               subnormal size is valid: every position more than a
 *               few thousand subnormal steps from the origin clamps)
 *   dims        host, in:    cells per axis, each in [1, 2^24]; the cell
 *               count C = dims[0]*dims[1]*dims[2] must be <= 2^32-2
 *   celdaDe     device, out: n u32, cell index of each particle (its key
 *               with UGP_FLAG_MORTON)
 *   conteos     device, out: K u32, particles per cell (the histogram;
 *               it still holds the histogram when the call completes);
 *               K = C unless UGP_FLAG_MORTON (ugp_grid_key_count())
 *   inicios     device, out: K+1 u32, exclusive prefix sum of conteos,
 *               inicios[K] = n
 *   ordenado    device, out: n u32, particle indices grouped by cell:
 *               cell c occupies [inicios[c], inicios[c+1])
 *   reordered   device, out: n records, reordered[k] = particles[ordenado[k]]
 *               bit for bit (unused, may be NULL, with UGP_FLAG_INDEX_ONLY);
 *               must not overlap particles (double buffer,
 *               page "Reordenar por celda...", section "El kernel de
 *               reordenación")
 *   workspace   device scratch of at least ugp_grid_workspace_bytes(); its
 *               content on entry is ignored and on exit unspecified
 *   flags       UGP_FLAG_* bits
 *   stream      hipStream_t or NULL
 *
 * Returns UGP_OK once all kernels are enqueued, or an error code with
 * nothing enqueued. Calls that share a workspace must be ordered on one
 * stream; calls on different streams need different workspaces. */
int ugp_grid_build(const ugp_particle *particles, uint32_t n, const float origin[3],
                   float cell_size, const uint32_t dims[3], uint32_t *celdaDe, uint32_t *conteos,
                   uint32_t *inicios, uint32_t *ordenado, ugp_particle *reordered, void *workspace,
                   size_t workspace_bytes, uint32_t flags, void *stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the same
 * build as ugp_grid_build() without a workspace argument. Its workspace is a
 * library-owned device array of UGP_NOALLOC_SCRATCH_BYTES on each GPU (held
 * from the library's load until the process ends); the call allocates and
 * frees nothing. Every call on one GPU shares that array, so calls that
 * overlap on one GPU (other streams, other host threads) race: order them
 * on one stream. Arguments, outputs and errors as ugp_grid_build();
 * UGP_ERR_WORKSPACE, with nothing enqueued, when ugp_grid_workspace_bytes()
 * for (n, dims, flags) exceeds UGP_NOALLOC_SCRATCH_BYTES (it covers, for
 * example, 1,000,000 particles on a 128^3 grid with any flags). */
#define UGP_NOALLOC_SCRATCH_BYTES (48u << 20)
int ugp_grid_build_noalloc(const ugp_particle *particles, uint32_t n, const float origin[3],
                           float cell_size, const uint32_t dims[3], uint32_t *celdaDe, uint32_t *conteos,
                           uint32_t *inicios, uint32_t *ordenado, ugp_particle *reordered, uint32_t flags,
                           void *stream);

/* Enqueue one stage slot (0..UGP_NUM_STAGES-1) of ugp_grid_build() with the
 * same arguments. Running the slots 0..UGP_NUM_STAGES-1 in order on one stream
 * is exactly ugp_grid_build(); a stage that does not apply to `flags`
 * returns UGP_OK and enqueues nothing. Each stage reads what the previous
 * ones left in the outputs and the workspace, so stages must run in order
 * with identical arguments. Intended for per-stage timing and tests. */
int ugp_grid_build_stage(uint32_t stage, const ugp_particle *particles, uint32_t n,
                         const float origin[3], float cell_size, const uint32_t dims[3],
                         uint32_t *celdaDe, uint32_t *conteos, uint32_t *inicios,
                         uint32_t *ordenado, ugp_particle *reordered, void *workspace,
                         size_t workspace_bytes, uint32_t flags, void *stream);

/* ugp_grid_build() plus the overflow diagnostics of page "Contar
 * partículas por celda", section "Detectar el desbordamiento sin salir de
 * la GPU", computed on the device in the same call:
 *   capacity  particles a cell may hold (any value; 0 makes every insertion
 *             an overflow)
 *   diag      device, out: 2 u32, 4-byte aligned, must not overlap any other
 *             buffer of the call.
 *             diag[0] = largest occupancy of any cell = max_c conteos[c]
 *                       (0 when n == 0);
 *             diag[1] = insertions that found their cell already holding
 *                       `capacity` or more particles
 *                     = sum_c max(0, conteos[c] - capacity).
 * Both are independent of the order of insertion. On the tile paths (up to
 * 2^26 keys) the reduction runs inside the tile kernel over its LDS
 * histogram (no extra memory traffic); on the global-atomic path a
 * reduction over conteos follows the scatter. Other arguments and errors as
 * ugp_grid_build(); UGP_ERR_NULL for a NULL diag. */
int ugp_grid_build_diag(const ugp_particle *particles, uint32_t n, const float origin[3],
                        float cell_size, const uint32_t dims[3], uint32_t *celdaDe,
                        uint32_t *conteos, uint32_t *inicios, uint32_t *ordenado,
                        ugp_particle *reordered, void *workspace, size_t workspace_bytes,
                        uint32_t capacity, uint32_t *diag, uint32_t flags, void *stream);

/* The same two diagnostics from an existing histogram (for example one
 * read back every few frames, as the page suggests):
 *   conteos   device, in: `cells` u32, 16-byte aligned (may be NULL when
 *             cells == 0)
 *   diag      device, out: 2 u32 as in ugp_grid_build_diag(), 4-byte
 *             aligned, must not overlap conteos.
 * One kernel launch: each workgroup reduces its part into a partial held in
 * a slot of a library-owned device array, and the last workgroup to finish
 * folds the partials into diag (no clear beforehand). Slots are dealt round
 * robin over 64, so up to 64 calls (also those inside ugp_grid_build_diag()
 * on the global-atomic path) may be in flight at once on one GPU.
 * Returns UGP_OK once enqueued, UGP_ERR_NULL / UGP_ERR_ALIGN /
 * UGP_ERR_ALIAS with nothing enqueued, or UGP_ERR_HIP. */
int ugp_cell_diag(const uint32_t *conteos, uint32_t cells, uint32_t capacity, uint32_t *diag,
                  void *stream);

/* ugp_cell_diag() with two caller-owned HIP events (hipEvent_t passed as
 * void*) recorded at its kernel's own start and end (hipExtLaunchKernel), so
 * their interval is the kernel's execution time. Returns UGP_ERR_ARG for a
 * NULL event (nothing enqueued); otherwise as ugp_cell_diag(), and on an
 * error the events are not recorded. Intended for per-kernel timing. */
int ugp_cell_diag_timed(const uint32_t *conteos, uint32_t cells, uint32_t capacity, uint32_t *diag,
                        void *stream, void *event_before, void *event_after);

/* A neighbour query that consumes a finished index: for each particle, the
 * number of other particles among the 27 cells around its cell whose
 * squared distance (dx*dx + dy*dy) + dz*dz (binary32, dx = xj - xi, no fused
 * multiply-add) is <= radius*radius. Page "Construir el índice...", section
 * "La dispersión" (walking a cell's slice), and page "Reordenar por
 * celda...", sections "Qué cuesta la indirección" and "El orden de las
 * celdas también importa" (the 27-cell loop; why the data order matters).
 * With radius <= cell_size and every particle inside the grid this counts
 * every neighbour within the radius; cells outside the grid are skipped.
 *
 *   particles  device, in: n records, 16-byte aligned. Either the build's
 *              input (original order; pass its ordenado) or the build's
 *              `reordered` output (cell order; pass ordenado = NULL).
 *   origin, cell_size, dims   as given to the build
 *   inicios    device, in: the build's K+1 starts (K = ugp_grid_key_count())
 *   ordenado   device, in: the build's n particle indices, or NULL (above)
 *   radius     finite, >= 0
 *   counts     device, out: n u32, counts[k] for particle k of `particles`
 *              (original index with ordenado; cell-order slot without);
 *              must not overlap the inputs. Queries are taken in cell
 *              order (with ordenado, the one at place k is particle
 *              ordenado[k]), so with ordenado every entry is written when
 *              ordenado is a permutation of 0..n-1, as the build leaves
 *              it; an entry >= n is skipped
 *   flags      0 or UGP_FLAG_MORTON, as in the build
 * Returns UGP_OK once enqueued; UGP_ERR_NULL / UGP_ERR_ARG / UGP_ERR_RANGE /
 * UGP_ERR_ALIGN / UGP_ERR_ALIAS with nothing enqueued; UGP_ERR_HIP. The
 * kernel reads inicios only at keys of in-grid cells and clips every slice
 * to n, so an inconsistent index cannot make it read out of bounds. */
int ugp_neighbor_count(const ugp_particle *particles, uint32_t n, const float origin[3],
                       float cell_size, const uint32_t dims[3], const uint32_t *inicios,
                       const uint32_t *ordenado, float radius, uint32_t *counts, uint32_t flags,
                       void *stream);

/* ugp_grid_build() with two caller-owned HIP events (hipEvent_t passed as
 * void*) that time stage slot `timed_stage`, in the same call, so no host
 * work separates the stages. When the slot is one kernel launch, the events
 * are recorded at that kernel's own start and end (hipExtLaunchKernel), so
 * their interval is the kernel's execution time, as a profiler's kernel
 * trace reports it; otherwise they are recorded on `stream` immediately
 * before and after the slot (a slot that enqueues nothing gives an empty
 * interval). Returns UGP_ERR_ARG for a bad slot or a NULL event; otherwise
 * as ugp_grid_build(). Intended for per-kernel timing. */
int ugp_grid_build_timed(const ugp_particle *particles, uint32_t n, const float origin[3],
                         float cell_size, const uint32_t dims[3], uint32_t *celdaDe,
                         uint32_t *conteos, uint32_t *inicios, uint32_t *ordenado,
                         ugp_particle *reordered, void *workspace, size_t workspace_bytes,
                         uint32_t flags, void *stream, uint32_t timed_stage, void *event_before,
                         void *event_after);

/* Name of stage slot `stage` for this problem shape and flags
 * ("chunk_sort", "count", ...), or NULL when the slot runs nothing or the shape is
 * invalid. Static storage. Pure host function. */
const char *ugp_grid_stage_name(uint32_t n, const uint32_t dims[3], uint32_t flags, uint32_t stage);

/* Bytes of device workspace ugp_exclusive_scan_u32() needs for `count`
 * elements. Pure host function. */
int ugp_scan_workspace_bytes(uint32_t count, size_t *bytes);

/* Exclusive prefix sum of `count` u32 values with the total appended:
 * out[0] = 0, out[i+1] = out[i] + in[i], out[count] = sum (mod 2^32).
 * Page "Construir el índice...", section "Del conteo al inicio".
 *   in   device, in:  count u32 (count may be 0: out[0] = 0)
 *   out  device, out: count+1 u32, must not overlap `in`
 *   workspace  device scratch of ugp_scan_workspace_bytes(count) bytes */
int ugp_exclusive_scan_u32(const uint32_t *in, uint32_t count, uint32_t *out, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Gather reorder on its own: dst[k] = src[idx[k]] for k < n, 32 bytes each,
 * bit for bit. Page "Reordenar por celda...", section "El kernel de
 * reordenación". Every idx[k] must be < n_src; the kernel checks and skips
 * (leaves dst[k] unwritten) any index that is not, and the call returns
 * UGP_OK regardless -- validate indices beforehand when they are untrusted.
 *   src  device, in: n_src records;  idx device, in: n u32;
 *   dst  device, out: n records, must not overlap src or idx. */
int ugp_reorder(const ugp_particle *src, uint32_t n_src, const uint32_t *idx, uint32_t n,
                ugp_particle *dst, void *stream);

/* One array of a split particle state for ugp_reorder_arrays(). */
typedef struct ugp_array_desc {
  const void *src;      /* device, in: n_src elements of elem_bytes */
  void *dst;            /* device, out: n elements of elem_bytes */
  uint32_t elem_bytes;  /* a multiple of 4 */
} ugp_array_desc;

/* Gather several arrays with one index in one kernel: for every array q and
 * k < n, dst_q[k] = src_q[idx[k]], elem_bytes_q bytes, bit for bit. Page
 * "Reordenar por celda...", section "El kernel de reordenación": a state
 * split over buffers (page "El estado de las partículas en storage
 * buffers", section "Array de estructuras o estructura de arrays": hot
 * kinematics and cold appearance) is reordered with the same ordenado,
 * read once for all arrays.
 *   idx     device, in: n u32; entries >= n_src are skipped (that dst
 *           element is left unwritten; the call still returns UGP_OK)
 *   arrays  host, in: `count` descriptors, 1 <= count <= 8; pointers 4-byte
 *           aligned; 16-byte element chunks are used when every size is a
 *           multiple of 16 and every pointer 16-byte aligned, 4-byte chunks
 *           otherwise; one element of all arrays together must fit 256
 *           chunks (up to 4096 bytes with 16-byte chunks, 1024 otherwise).
 *           No dst may overlap idx, any src, or another dst.
 * Returns UGP_OK once enqueued, UGP_ERR_ARG / UGP_ERR_NULL / UGP_ERR_ALIGN /
 * UGP_ERR_ALIAS with nothing enqueued, or UGP_ERR_HIP. */
int ugp_reorder_arrays(const uint32_t *idx, uint32_t n, uint32_t n_src,
                       const ugp_array_desc *arrays, uint32_t count, void *stream);

/* Human-readable text for a status code (static storage, never NULL). */
const char *ugp_status_string(int status);

/* ABI version of this header: 1. */
int ugp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* UGP_H */
