/*
 * ugp_oracle.c -- plain, sequential CPU oracle for the uniform-grid index
 * build (count -> scan -> scatter -> reorder).
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library. The GPU library shares
 * no code, header, table or constant with it, and the product path never
 * calls it.
 *
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fPIC -shared
 * On x86-64 every float operation below is one IEEE-754 binary32 operation
 * rounded to nearest-even (SSE arithmetic, no excess precision), and the
 * division is the correctly rounded one.
 *
 * What it follows, page by page (titles and sections of the source pages):
 *
 *  - "Contar partículas por celda", section "El kernel": each particle's
 *    cell index is computed once, stored per particle (celdaDe), and
 *    counted into a per-cell histogram (conteos). The cell function does
 *    one floor, a division per axis and two multiplications for the
 *    linear index, and the range clamp lives inside the index function.
 *    The page takes the function bodies from an earlier lesson it does
 *    not reproduce, so the rule written out below is the plainest reading
 *    the pages support: per axis floor((p - o) / h), clamped to
 *    [0, dim - 1], then x + y*nx + z*nx*ny (that linear order is stated on
 *    "Reordenar por celda y la coalescencia de memoria", section
 *    "El orden de las celdas también importa").
 *  - "Construir el índice de la rejilla con un prefix sum":
 *      section "Del conteo al inicio" -- inicios is the exclusive prefix
 *      sum of conteos, with one extra trailing slot that holds the total;
 *      section "La dispersión" -- a per-cell cursor starting at zero hands
 *      out slots inicios[c] + cursor[c] and each particle index is written
 *      there (ordenado);
 *      section "El orden dentro de la celda" -- the stable order within a
 *      cell uses the particle index as the tie-break, which is what the
 *      sequential loop below produces.
 *  - "Reordenar por celda y la coalescencia de memoria", section
 *    "El kernel de reordenación": a gather, destination slot k receives
 *    the whole 32-byte record of particle ordenado[k].
 *  - "Contar partículas por celda", section "Detectar el desbordamiento
 *    sin salir de la GPU": the diagnostic pair (largest per-cell occupancy,
 *    number of insertions that found the cell already at or above a fixed
 *    capacity) -- computed here in closed form from the histogram.
 *  - "Reordenar por celda y la coalescencia de memoria", section "El orden
 *    de las celdas también importa": cells may instead be numbered along
 *    the Z (Morton) curve. The page gives no formula; the reading taken is
 *    the textbook 3-D bit interleave of the clamped cell coordinates --
 *    bit b of x, y, z goes to key bits 3b, 3b+1, 3b+2 -- with every axis
 *    padded to B bits, 2^B being the smallest power of two >= the largest
 *    dimension, so there are 2^(3B) keys (exactly the cell count on a cubic
 *    power-of-two grid; other grids leave keys no cell maps to).
 *  - "Construir el índice de la rejilla con un prefix sum", section "La
 *    dispersión" (walking one cell's slice), and "Reordenar por celda y la
 *    coalescencia de memoria", section "El orden de las celdas también
 *    importa" (the neighbour loop visits the 27 cells around a particle's
 *    cell): a neighbour query that consumes the index. The pages give no
 *    kernel for it; the reading taken is a neighbour count -- for each
 *    particle, the other particles in the 27 cells around its (clamped)
 *    cell whose squared distance is <= radius^2, the squared distance being
 *    (dx*dx + dy*dy) + dz*dz in binary32 with dx = xj - xi. With radius <=
 *    cell size and every particle inside the grid this is every neighbour
 *    within the radius.
 *  - "Reordenar por celda y la coalescencia de memoria", section "El kernel
 *    de reordenación": when the state is split over several buffers, every
 *    buffer is gathered with the same ordenado; the oracle gathers any
 *    element size byte for byte.
 */
#include <float.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define UGPO_OK 0
#define UGPO_ERR_NULL (-1)
#define UGPO_ERR_ARG (-2)
#define UGPO_ERR_RANGE (-3)

/* largest per-axis dimension: dim - 1 must be exact in float32 */
#define UGPO_MAX_DIM (1u << 24)

/* cell numbering */
#define UGPO_ORDER_LINEAR 0u
#define UGPO_ORDER_MORTON 1u
/* Morton keys: at most 10 bits per axis, 2^30 keys */
#define UGPO_MORTON_MAX_BITS 10u

/* ------------------------------------------------------------------ */
/* Argument checks (the oracle rejects what it cannot define).          */
/* ------------------------------------------------------------------ */

int ugp_oracle_check_grid(const float origin[3], float cell_size, const uint32_t dims[3],
                          uint64_t *cells_out) {
    if (!origin || !dims) return UGPO_ERR_NULL;
    /* a usable cell size is any finite positive float, subnormal ones
       included: the division and the clamp are defined for all of them */
    if (!isfinite(cell_size) || !(cell_size > 0.0f)) return UGPO_ERR_ARG;
    for (int a = 0; a < 3; ++a) {
        if (!isfinite(origin[a])) return UGPO_ERR_ARG;
        if (dims[a] < 1u || dims[a] > UGPO_MAX_DIM) return UGPO_ERR_RANGE;
    }
    uint64_t cells = (uint64_t)dims[0] * (uint64_t)dims[1] * (uint64_t)dims[2];
    if (cells > (uint64_t)UINT32_MAX - 1u) return UGPO_ERR_RANGE;
    if (cells_out) *cells_out = cells;
    return UGPO_OK;
}

/* ------------------------------------------------------------------ */
/* Step 1a: the cell of one coordinate.                                 */
/* ------------------------------------------------------------------ */

/* One axis: subtract the origin (one rounding), divide by the cell size
 * (one correctly rounded division), floor, then clamp into [0, dim-1].
 * The clamp is done on the float value before any conversion: the lower
 * test is written so that NaN fails it (NaN and -inf go to 0), the upper
 * test sends +inf and everything past the last face to dim-1. */
static uint32_t oracle_axis_cell(float p, float o, float h, uint32_t dim) {
    float t = p - o;
    float q = t / h;
    float f = floorf(q);
    if (!(f >= 0.0f)) f = 0.0f;
    float top = (float)(dim - 1u);
    if (f > top) f = top;
    return (uint32_t)f;
}

/* Morton keys: bits per axis and key count for a grid. */
int ugp_oracle_morton_bits(const uint32_t dims[3], uint32_t *bits, uint64_t *keys) {
    if (!dims || !bits) return UGPO_ERR_NULL;
    uint32_t largest = 0;
    for (int a = 0; a < 3; ++a) {
        if (dims[a] < 1u || dims[a] > UGPO_MAX_DIM) return UGPO_ERR_RANGE;
        if (dims[a] > largest) largest = dims[a];
    }
    uint32_t b = 0;
    while ((1u << b) < largest) ++b;
    if (b > UGPO_MORTON_MAX_BITS) return UGPO_ERR_RANGE;
    *bits = b;
    if (keys) *keys = 1ull << (3u * b);
    return UGPO_OK;
}

/* The Morton key of cell (kx, ky, kz), bit by bit. */
uint32_t ugp_oracle_morton_key(uint32_t kx, uint32_t ky, uint32_t kz, uint32_t bits) {
    uint64_t key = 0;
    for (uint32_t b = 0; b < bits; ++b) {
        key |= (uint64_t)((kx >> b) & 1u) << (3u * b);
        key |= (uint64_t)((ky >> b) & 1u) << (3u * b + 1u);
        key |= (uint64_t)((kz >> b) & 1u) << (3u * b + 2u);
    }
    return (uint32_t)key;
}

/* Array form: k3 holds n (kx, ky, kz) triples. */
int ugp_oracle_morton_keys(const uint32_t *k3, uint32_t n, uint32_t bits, uint32_t *out) {
    if (n > 0 && (!k3 || !out)) return UGPO_ERR_NULL;
    if (bits > UGPO_MORTON_MAX_BITS) return UGPO_ERR_RANGE;
    for (uint32_t i = 0; i < n; ++i)
        out[i] = ugp_oracle_morton_key(k3[3u * i], k3[3u * i + 1u], k3[3u * i + 2u], bits);
    return UGPO_OK;
}

/* Number of cell keys of a grid under a numbering (linear: the cell count). */
int ugp_oracle_key_count(const float origin[3], float cell_size, const uint32_t dims[3],
                         uint32_t order, uint64_t *keys) {
    uint64_t cells = 0;
    int st = ugp_oracle_check_grid(origin, cell_size, dims, &cells);
    if (st != UGPO_OK) return st;
    if (order == UGPO_ORDER_LINEAR) {
        if (keys) *keys = cells;
        return UGPO_OK;
    }
    if (order != UGPO_ORDER_MORTON) return UGPO_ERR_ARG;
    uint32_t bits = 0;
    return ugp_oracle_morton_bits(dims, &bits, keys);
}

/* Step 1b: per-particle cell key. Linear order: x + y*nx + z*nx*ny;
 * Morton order: the interleave above.
 * particles: n records of 8 floats, position in floats 0..2. */
int ugp_oracle_cell_key(const float *particles, uint32_t n, const float origin[3],
                        float cell_size, const uint32_t dims[3], uint32_t order,
                        uint32_t *celdaDe) {
    uint64_t cells = 0;
    int st = ugp_oracle_key_count(origin, cell_size, dims, order, &cells);
    if (st != UGPO_OK) return st;
    uint32_t bits = 0;
    if (order == UGPO_ORDER_MORTON) ugp_oracle_morton_bits(dims, &bits, NULL);
    if (n > 0 && (!particles || !celdaDe)) return UGPO_ERR_NULL;
    const uint64_t nx = dims[0];
    const uint64_t nxy = (uint64_t)dims[0] * (uint64_t)dims[1];
    for (uint32_t i = 0; i < n; ++i) {
        const float *rec = particles + (size_t)i * 8u;
        uint64_t kx = oracle_axis_cell(rec[0], origin[0], cell_size, dims[0]);
        uint64_t ky = oracle_axis_cell(rec[1], origin[1], cell_size, dims[1]);
        uint64_t kz = oracle_axis_cell(rec[2], origin[2], cell_size, dims[2]);
        uint64_t c;
        if (order == UGPO_ORDER_MORTON) {
            c = ugp_oracle_morton_key((uint32_t)kx, (uint32_t)ky, (uint32_t)kz, bits);
        } else {
            c = kx + ky * nx + kz * nxy;
        }
        if (c >= cells) return UGPO_ERR_RANGE; /* cannot happen after the clamp */
        celdaDe[i] = (uint32_t)c;
    }
    return UGPO_OK;
}

/* Linear cell index (the default numbering). */
int ugp_oracle_cell_index(const float *particles, uint32_t n, const float origin[3],
                          float cell_size, const uint32_t dims[3], uint32_t *celdaDe) {
    return ugp_oracle_cell_key(particles, n, origin, cell_size, dims, UGPO_ORDER_LINEAR, celdaDe);
}

/* ------------------------------------------------------------------ */
/* Step 1c: histogram of cell indices.                                  */
/* ------------------------------------------------------------------ */

int ugp_oracle_histogram(const uint32_t *celdaDe, uint32_t n, uint32_t cells,
                         uint32_t *conteos) {
    if (cells > 0 && !conteos) return UGPO_ERR_NULL;
    if (n > 0 && !celdaDe) return UGPO_ERR_NULL;
    for (uint32_t c = 0; c < cells; ++c) conteos[c] = 0u;
    for (uint32_t i = 0; i < n; ++i) {
        uint32_t c = celdaDe[i];
        if (c >= cells) return UGPO_ERR_RANGE;
        conteos[c] += 1u;
    }
    return UGPO_OK;
}

/* ------------------------------------------------------------------ */
/* Step 2: exclusive prefix sum with the total in slot `cells`.         */
/* ------------------------------------------------------------------ */

int ugp_oracle_exclusive_scan(const uint32_t *conteos, uint32_t cells, uint32_t *inicios) {
    if (!inicios) return UGPO_ERR_NULL;
    if (cells > 0 && !conteos) return UGPO_ERR_NULL;
    uint64_t run = 0;
    for (uint32_t c = 0; c < cells; ++c) {
        inicios[c] = (uint32_t)run;
        run += conteos[c];
        if (run > UINT32_MAX) return UGPO_ERR_RANGE;
    }
    inicios[cells] = (uint32_t)run;
    return UGPO_OK;
}

/* ------------------------------------------------------------------ */
/* Step 3: scatter with a per-cell cursor, particles taken in ascending  */
/* index order, so each cell lists its particles in ascending order.     */
/* `cursor` is caller scratch of `cells` entries.                       */
/* ------------------------------------------------------------------ */

int ugp_oracle_scatter(const uint32_t *celdaDe, uint32_t n, const uint32_t *inicios,
                       uint32_t cells, uint32_t *cursor, uint32_t *ordenado) {
    if (n == 0) return UGPO_OK;
    if (!celdaDe || !inicios || !cursor || !ordenado) return UGPO_ERR_NULL;
    for (uint32_t c = 0; c < cells; ++c) cursor[c] = 0u;
    for (uint32_t i = 0; i < n; ++i) {
        uint32_t c = celdaDe[i];
        if (c >= cells) return UGPO_ERR_RANGE;
        uint64_t slot = (uint64_t)inicios[c] + cursor[c];
        if (slot >= inicios[c + 1] || slot >= n) return UGPO_ERR_RANGE;
        ordenado[slot] = i;
        cursor[c] += 1u;
    }
    return UGPO_OK;
}

/* ------------------------------------------------------------------ */
/* Step 4: gather reorder, 32 bytes copied verbatim per record.         */
/* ------------------------------------------------------------------ */

int ugp_oracle_reorder(const float *particles, const uint32_t *ordenado, uint32_t n,
                       float *reordered) {
    if (n == 0) return UGPO_OK;
    if (!particles || !ordenado || !reordered) return UGPO_ERR_NULL;
    for (uint32_t k = 0; k < n; ++k) {
        uint32_t src = ordenado[k];
        if (src >= n) return UGPO_ERR_RANGE;
        memcpy(reordered + (size_t)k * 8u, particles + (size_t)src * 8u, 32u);
    }
    return UGPO_OK;
}

/* ------------------------------------------------------------------ */
/* The whole chain.  cursor: caller scratch of `keys` entries, where     */
/* keys is the key count of the numbering (ugp_oracle_key_count).        */
/* ------------------------------------------------------------------ */

int ugp_oracle_grid_build_keyed(const float *particles, uint32_t n, const float origin[3],
                                float cell_size, const uint32_t dims[3], uint32_t order,
                                uint32_t *celdaDe, uint32_t *conteos, uint32_t *inicios,
                                uint32_t *ordenado, float *reordered, uint32_t *cursor) {
    uint64_t cells64 = 0;
    int st = ugp_oracle_key_count(origin, cell_size, dims, order, &cells64);
    if (st != UGPO_OK) return st;
    uint32_t cells = (uint32_t)cells64;
    st = ugp_oracle_cell_key(particles, n, origin, cell_size, dims, order, celdaDe);
    if (st != UGPO_OK) return st;
    st = ugp_oracle_histogram(celdaDe, n, cells, conteos);
    if (st != UGPO_OK) return st;
    st = ugp_oracle_exclusive_scan(conteos, cells, inicios);
    if (st != UGPO_OK) return st;
    st = ugp_oracle_scatter(celdaDe, n, inicios, cells, cursor, ordenado);
    if (st != UGPO_OK) return st;
    return ugp_oracle_reorder(particles, ordenado, n, reordered);
}

int ugp_oracle_grid_build(const float *particles, uint32_t n, const float origin[3],
                          float cell_size, const uint32_t dims[3], uint32_t *celdaDe,
                          uint32_t *conteos, uint32_t *inicios, uint32_t *ordenado,
                          float *reordered, uint32_t *cursor) {
    return ugp_oracle_grid_build_keyed(particles, n, origin, cell_size, dims, UGPO_ORDER_LINEAR,
                                       celdaDe, conteos, inicios, ordenado, reordered, cursor);
}

/* ------------------------------------------------------------------ */
/* Overflow diagnostics, closed form from the histogram.                 */
/* Insertion number j (1-based) into cell c overflows when j > capacity, */
/* so cell c contributes max(0, conteos[c] - capacity) overflows and the */
/* largest occupancy is the largest count.                               */
/* ------------------------------------------------------------------ */

int ugp_oracle_diag(const uint32_t *conteos, uint32_t cells, uint32_t capacity,
                    uint32_t *max_per_cell, uint32_t *overflows) {
    if (!max_per_cell || !overflows) return UGPO_ERR_NULL;
    if (cells > 0 && !conteos) return UGPO_ERR_NULL;
    uint32_t mx = 0;
    uint64_t ov = 0;
    for (uint32_t c = 0; c < cells; ++c) {
        uint32_t v = conteos[c];
        if (v > mx) mx = v;
        if (v > capacity) ov += (uint64_t)(v - capacity);
    }
    *max_per_cell = mx;
    *overflows = (uint32_t)ov;
    return UGPO_OK;
}

/* ------------------------------------------------------------------ */
/* Neighbour count over the 27 cells around each particle's cell.       */
/* index: the keyed build of the same particles (inicios, ordenado).    */
/* counts[i] for particle i, in the original order.                     */
/* ------------------------------------------------------------------ */

int ugp_oracle_neighbor_count(const float *particles, uint32_t n, const float origin[3],
                              float cell_size, const uint32_t dims[3], uint32_t order,
                              const uint32_t *inicios, const uint32_t *ordenado, float radius,
                              uint32_t *counts) {
    uint64_t keys = 0;
    int st = ugp_oracle_key_count(origin, cell_size, dims, order, &keys);
    if (st != UGPO_OK) return st;
    if (!isfinite(radius) || !(radius >= 0.0f)) return UGPO_ERR_ARG;
    if (n == 0) return UGPO_OK;
    if (!particles || !inicios || !ordenado || !counts) return UGPO_ERR_NULL;
    uint32_t bits = 0;
    if (order == UGPO_ORDER_MORTON) ugp_oracle_morton_bits(dims, &bits, NULL);
    const float r2 = radius * radius;
    for (uint32_t i = 0; i < n; ++i) {
        const float *pi = particles + (size_t)i * 8u;
        int64_t k[3];
        for (int a = 0; a < 3; ++a) k[a] = oracle_axis_cell(pi[a], origin[a], cell_size, dims[a]);
        uint32_t count = 0;
        for (int64_t z = k[2] - 1; z <= k[2] + 1; ++z) {
            if (z < 0 || z >= (int64_t)dims[2]) continue;
            for (int64_t y = k[1] - 1; y <= k[1] + 1; ++y) {
                if (y < 0 || y >= (int64_t)dims[1]) continue;
                for (int64_t x = k[0] - 1; x <= k[0] + 1; ++x) {
                    if (x < 0 || x >= (int64_t)dims[0]) continue;
                    uint64_t c;
                    if (order == UGPO_ORDER_MORTON)
                        c = ugp_oracle_morton_key((uint32_t)x, (uint32_t)y, (uint32_t)z, bits);
                    else
                        c = (uint64_t)x + (uint64_t)y * dims[0] + (uint64_t)z * dims[0] * dims[1];
                    if (c >= keys) return UGPO_ERR_RANGE;
                    for (uint32_t t = inicios[c]; t < inicios[c + 1]; ++t) {
                        const uint32_t j = ordenado[t];
                        if (j >= n) return UGPO_ERR_RANGE;
                        if (j == i) continue;
                        const float *pj = particles + (size_t)j * 8u;
                        const float dx = pj[0] - pi[0];
                        const float dy = pj[1] - pi[1];
                        const float dz = pj[2] - pi[2];
                        const float d2 = dx * dx + dy * dy + dz * dz;
                        if (d2 <= r2) count += 1u;
                    }
                }
            }
        }
        counts[i] = count;
    }
    return UGPO_OK;
}

/* ------------------------------------------------------------------ */
/* Gather of one array of fixed-size elements: dst[k] = src[idx[k]],     */
/* elem_bytes bytes each, for k < n (every idx[k] < n_src).              */
/* ------------------------------------------------------------------ */

int ugp_oracle_gather_bytes(const void *src, uint32_t n_src, uint32_t elem_bytes,
                            const uint32_t *idx, uint32_t n, void *dst) {
    if (n == 0) return UGPO_OK;
    if (!src || !idx || !dst) return UGPO_ERR_NULL;
    if (elem_bytes == 0) return UGPO_ERR_ARG;
    const unsigned char *s = (const unsigned char *)src;
    unsigned char *d = (unsigned char *)dst;
    for (uint32_t k = 0; k < n; ++k) {
        if (idx[k] >= n_src) return UGPO_ERR_RANGE;
        memcpy(d + (size_t)k * elem_bytes, s + (size_t)idx[k] * elem_bytes, elem_bytes);
    }
    return UGPO_OK;
}
