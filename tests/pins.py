"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each ``pin_*`` function takes an oracle object (the default build, or a
deliberately broken copy in the mutation test) and raises AssertionError
when the oracle disagrees with an independent source of truth:

* the worked example printed on "Construir el índice de la rejilla con un
  prefix sum", section "Del conteo al inicio" (golden fixture);
* exact rational arithmetic with an explicit IEEE binary32
  round-to-nearest-even written here from the definition of the format;
* hand-placed particles whose cell is known by construction;
* library routines the result must reduce to (``numpy.bincount``, a
  stable ``numpy.argsort``, fancy indexing);
* brute force over all cells on small inputs.
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# IEEE-754 binary32 rounding of an exact rational (round to nearest, ties to
# even), written from the format's definition: 24-bit significand, smallest
# normal exponent -126, subnormal spacing 2^-149, overflow to infinity.
# ---------------------------------------------------------------------------

def round_f32(x: Fraction):
    if x == 0:
        return Fraction(0)
    neg = x < 0
    a = -x if neg else x
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # normalise so that 2^e <= a < 2^(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e, -126) - 23  # exponent of one unit in the last place
    scaled = a / (Fraction(2) ** q)
    m = scaled.numerator // scaled.denominator
    r = scaled - m
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and m % 2 == 1):
        m += 1
    val = m * (Fraction(2) ** q)
    if val >= Fraction(2) ** 128:
        return -math.inf if neg else math.inf
    return -val if neg else val


def model_axis_cell(p: float, o: float, h: float, dim: int) -> int:
    """Cell along one axis by exact rationals plus explicit binary32 rounding.

    t = round(p - o); q = round(t / h); floor; clamp to [0, dim - 1].
    NaN and -inf go to 0, +inf to dim - 1.
    """
    if math.isnan(p):
        return 0
    if math.isinf(p):
        return 0 if p < 0 else dim - 1
    t = round_f32(Fraction(p) - Fraction(o))
    if isinstance(t, float):  # overflowed to +-inf
        return 0 if t < 0 else dim - 1
    q = round_f32(t / Fraction(h))
    if isinstance(q, float):
        return 0 if q < 0 else dim - 1
    f = math.floor(q)
    if f < 0:
        return 0
    if f > dim - 1:
        return dim - 1
    return int(f)


def model_cell_index(particles, origin, h, dims) -> np.ndarray:
    """Linear index x + y*nx + z*nx*ny of the binary32 model, one particle at a time."""
    p = np.asarray(particles, dtype=np.float32).reshape(-1, 8)
    o = [float(v) for v in np.asarray(origin, dtype=np.float32)]
    hh = float(np.float32(h))
    d = [int(v) for v in dims]
    out = np.empty(p.shape[0], dtype=np.uint64)
    for i in range(p.shape[0]):
        k = [model_axis_cell(float(p[i, a]), o[a], hh, d[a]) for a in range(3)]
        out[i] = k[0] + k[1] * d[0] + k[2] * d[0] * d[1]
    return out


# ---------------------------------------------------------------------------
# Pins
# ---------------------------------------------------------------------------

def pin_round_f32_helper():
    """The rounding helper itself against NumPy's double -> float32 cast."""
    rng = np.random.Generator(np.random.PCG64(99))
    xs = np.concatenate([
        rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 39, 2000),
        np.array([1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, 2.0 ** -149 * 1.5, 2.0 ** -150, 3.4028235e38]),
    ])
    for x in xs:
        x = float(x)
        want = float(np.float32(x))
        got = round_f32(Fraction(x))
        got = float(got)
        assert got == want or (math.isinf(want) and math.isinf(got)), (x, got, want)


def pin_worked_example_scan(orc):
    g = load_golden("worked_example_scan.json")
    inicios = orc.exclusive_scan(np.asarray(g["conteos"], dtype=np.uint32))
    assert inicios.tolist() == g["inicios_with_total_slot"], inicios.tolist()
    assert inicios[:-1].tolist() == g["inicios_printed"]
    # the end of cell c is the start of cell c+1 (trailing slot holds the total)
    assert inicios[1:].tolist() == g["finales_printed"]
    for c in g["empty_cells"]:
        assert inicios[c] == inicios[c + 1]


def pin_worked_example_pipeline(orc):
    """The printed example realised as particles and run through every step."""
    g = load_golden("worked_example_scan.json")
    conteos = g["conteos"]
    wl = W.make_worked_example(conteos, seed=7)
    r = orc.grid_build(wl.particles, wl.origin, wl.cell_size, wl.dims)
    assert r.conteos.tolist() == conteos
    assert r.inicios.tolist() == g["inicios_with_total_slot"]
    # vida holds each record's cell number by construction
    cell_of = wl.particles[:, 3].astype(np.int64)
    assert r.celdaDe.tolist() == cell_of.tolist()
    starts = g["inicios_with_total_slot"]
    for c in range(len(conteos)):
        sl = r.ordenado[starts[c]:starts[c + 1]]
        assert sorted(sl.tolist()) == sorted(np.nonzero(cell_of == c)[0].tolist())
        assert sl.tolist() == sorted(sl.tolist())  # stable: ascending particle index
        assert np.all(r.reordered[starts[c]:starts[c + 1], 3] == float(c))


def pin_cell_centres_noncubic(orc):
    """A particle at the centre of cell (kx, ky, kz) lands in kx + ky*nx + kz*nx*ny."""
    for dims in ((7, 5, 3), (1, 1, 1), (3, 1, 4), (2, 9, 1), (16, 16, 16)):
        ks = np.stack(np.meshgrid(*[np.arange(d) for d in dims], indexing="ij"), -1).reshape(-1, 3)
        for origin, h in (((0.0, 0.0, 0.0), 1.0), ((-5.0, 2.5, -0.75), 0.625), ((3.0, -1.0, 7.0), 0.0390625)):
            wl = W.make_cell_centres(dims, origin, h, ks)
            got = orc.cell_index(wl.particles, wl.origin, wl.cell_size, wl.dims)
            want = ks[:, 0] + ks[:, 1] * dims[0] + ks[:, 2] * dims[0] * dims[1]
            assert np.array_equal(got.astype(np.int64), want.astype(np.int64)), (dims, origin, h)


def pin_special_positions(orc):
    """Faces, outside points, NaN and infinities, by the clamp reading."""
    dims = np.array([7, 5, 3], dtype=np.uint32)
    o = np.array([-1.0, 2.0, 0.5], dtype=np.float32)
    h = np.float32(0.5)
    cases = []  # (x, y, z, expected (kx, ky, kz))
    cases.append((o[0] + 0.0, o[1] + 0.0, o[2] + 0.0, (0, 0, 0)))  # lower corner
    cases.append((o[0] + 1 * h, o[1] + 2 * h, o[2] + 1 * h, (1, 2, 1)))  # interior faces -> upper cell
    cases.append((o[0] + 7 * h, o[1] + 5 * h, o[2] + 3 * h, (6, 4, 2)))  # upper faces -> last cell
    cases.append((o[0] - 0.25, o[1] - 100.0, o[2] - 1e30, (0, 0, 0)))  # below -> 0
    cases.append((o[0] + 1e6, o[1] + 1e30, 3.0e38, (6, 4, 2)))  # above -> last
    cases.append((np.nan, np.nan, np.nan, (0, 0, 0)))
    cases.append((-np.inf, -np.inf, -np.inf, (0, 0, 0)))
    cases.append((np.inf, np.inf, np.inf, (6, 4, 2)))
    cases.append((np.inf, np.nan, -np.inf, (6, 0, 0)))
    cases.append((-0.0 + o[0], o[1] + 4.75 * h, o[2] + 2.999 * h, (0, 4, 2)))
    parts = np.zeros((len(cases), 8), dtype=np.float32)
    for i, c in enumerate(cases):
        parts[i, 0:3] = np.asarray(c[:3], dtype=np.float32)
    want = [k[0] + k[1] * 7 + k[2] * 35 for (_, _, _, k) in cases]
    got = orc.cell_index(parts, o, h, dims)
    assert got.tolist() == want, (got.tolist(), want)


def pin_binary32_model(orc, wl):
    """Oracle cell index equals the exact-rational binary32 model, every particle."""
    got = orc.cell_index(wl.particles, wl.origin, wl.cell_size, wl.dims)
    want = model_cell_index(wl.particles, wl.origin, wl.cell_size, wl.dims)
    bad = np.nonzero(got.astype(np.uint64) != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first at {bad[:5]}"


def pin_exact_floor_far_from_faces(orc, wl):
    """Away from cell faces the cell is the exact floor((p - o) / h), clamped."""
    p = wl.particles
    got = orc.cell_index(p, wl.origin, wl.cell_size, wl.dims)
    d = [int(v) for v in wl.dims]
    h = Fraction(float(wl.cell_size))
    checked = 0
    for i in range(p.shape[0]):
        ks = []
        far = True
        for a in range(3):
            q = (Fraction(float(p[i, a])) - Fraction(float(wl.origin[a]))) / h
            fl = math.floor(q)
            if min(q - fl, fl + 1 - q) < Fraction(1, 10_000):
                far = False
                break
            ks.append(min(max(fl, 0), d[a] - 1))
        if not far:
            continue
        checked += 1
        want = ks[0] + ks[1] * d[0] + ks[2] * d[0] * d[1]
        assert int(got[i]) == want, (i, p[i, :3], int(got[i]), want)
    assert checked > 0.9 * p.shape[0] or p.shape[0] < 100


def check_index_invariants(wl, r, stable: bool, keys: int | None = None):
    """Invariants every correct build satisfies (any size). `keys`: the key
    count when cells are numbered other than linearly (Morton)."""
    n = wl.n
    cells = wl.cells if keys is None else keys
    assert r.conteos.shape == (cells,)
    assert r.inicios.shape == (cells + 1,)
    assert int(r.inicios[0]) == 0
    assert int(r.inicios[-1]) == n  # trailing slot holds the total
    assert int(r.conteos.sum(dtype=np.uint64)) == n
    assert np.all(np.diff(r.inicios.astype(np.int64)) == r.conteos.astype(np.int64))
    # empty cell <=> start == end
    assert np.array_equal(r.conteos == 0, r.inicios[:-1] == r.inicios[1:])
    # ordenado is a permutation of 0..n-1
    seen = np.zeros(n, dtype=bool)
    seen[r.ordenado] = True
    assert seen.all()
    # slot k lies in the slice of its particle's cell
    k = np.arange(n, dtype=np.int64)
    c = r.celdaDe[r.ordenado].astype(np.int64)
    assert np.all(r.inicios[c] <= k) and np.all(k < r.inicios[c + 1])
    # reorder identity, bytewise
    assert np.array_equal(
        r.reordered.view(np.uint32), wl.particles.view(np.uint32)[r.ordenado]
    )
    if stable:
        assert np.array_equal(r.ordenado, np.argsort(r.celdaDe, kind="stable").astype(np.uint32))


def pin_library_reductions(orc, wl):
    """Histogram == bincount; stable scatter == stable argsort; gather == fancy index."""
    r = orc.grid_build(wl.particles, wl.origin, wl.cell_size, wl.dims)
    assert np.array_equal(r.conteos, np.bincount(r.celdaDe, minlength=wl.cells).astype(np.uint32))
    assert np.array_equal(r.inicios[:-1], (np.cumsum(r.conteos, dtype=np.uint64) - r.conteos).astype(np.uint32))
    assert np.array_equal(r.ordenado, np.argsort(r.celdaDe, kind="stable").astype(np.uint32))
    assert np.array_equal(r.reordered, wl.particles[r.ordenado])
    check_index_invariants(wl, r, stable=True)
    return r


def pin_brute_force_slices(orc, wl):
    """Every cell's slice equals {i : cell(i) = c}, found by visiting every cell."""
    r = orc.grid_build(wl.particles, wl.origin, wl.cell_size, wl.dims)
    key = model_cell_index(wl.particles, wl.origin, wl.cell_size, wl.dims) if wl.n <= 5000 else r.celdaDe
    key = np.asarray(key, dtype=np.int64)
    for c in range(wl.cells):
        members = np.nonzero(key == c)[0].tolist()  # visits every particle for every cell
        sl = r.ordenado[r.inicios[c]:r.inicios[c + 1]].tolist()
        assert sl == members, c


def pin_diag_closed_form(orc):
    """Overflow diagnostics against a replay of the per-insertion rule.

    The rule ("Contar partículas por celda", section "Detectar el
    desbordamiento sin salir de la GPU"): the counter's old value plus one
    is the occupancy after an insertion; the maximum of those is tracked
    and every insertion whose occupancy exceeds the capacity is counted.
    """
    rng = np.random.Generator(np.random.PCG64(5))
    for cells, n, cap in ((6, 15, 2), (50, 400, 8), (1, 30, 64), (300, 0, 4), (40, 500, 0)):
        keys = rng.integers(0, cells, n) if n else np.zeros(0, dtype=np.int64)
        occ = [0] * cells
        mx = 0
        ov = 0
        for c in keys:
            prev = occ[c]
            occ[c] = prev + 1
            mx = max(mx, prev + 1)
            if prev + 1 > cap:
                ov += 1
        got = orc.diag(np.asarray(occ, dtype=np.uint32), cap)
        assert got == (mx, ov), (cells, n, cap, got, (mx, ov))
    g = load_golden("worked_example_scan.json")
    assert orc.diag(np.asarray(g["conteos"], dtype=np.uint32), 2) == (5, 1 + 3 + 0 + 0 + 2)


def pin_grid_validation(orc):
    ok = (np.zeros(3, np.float32), np.float32(1.0), np.array([4, 4, 4], np.uint32))
    assert orc.check_grid(*ok) == 0
    assert orc.check_grid(ok[0], np.float32(0.0), ok[2]) != 0
    assert orc.check_grid(ok[0], np.float32(-1.0), ok[2]) != 0
    assert orc.check_grid(ok[0], np.float32(np.nan), ok[2]) != 0
    assert orc.check_grid(ok[0], np.float32(np.inf), ok[2]) != 0
    assert orc.check_grid(ok[0], np.float32(-0.0), ok[2]) != 0
    assert orc.check_grid(ok[0], np.float32(1e-40), ok[2]) == 0  # subnormal cell size
    assert orc.check_grid(ok[0], np.float32(1.4e-45), ok[2]) == 0  # the smallest subnormal
    assert orc.check_grid(ok[0], np.float32(1.1754944e-38), ok[2]) == 0  # smallest normal
    assert orc.check_grid(np.array([0, np.nan, 0], np.float32), ok[1], ok[2]) != 0
    assert orc.check_grid(ok[0], ok[1], np.array([0, 4, 4], np.uint32)) != 0
    assert orc.check_grid(ok[0], ok[1], np.array([1 << 24, 1, 1], np.uint32)) == 0
    assert orc.check_grid(ok[0], ok[1], np.array([(1 << 24) + 1, 1, 1], np.uint32)) != 0
    assert orc.check_grid(ok[0], ok[1], np.array([1 << 16, 1 << 16, 1], np.uint32)) != 0  # 2^32 cells
    assert orc.check_grid(ok[0], ok[1], np.array([65535, 65537, 1], np.uint32)) != 0  # 2^32 - 1 cells
    assert orc.check_grid(ok[0], ok[1], np.array([65535, 65536, 1], np.uint32)) == 0  # 2^32 - 2^16 cells


def pin_empty_and_degenerate(orc):
    # n = 0: histogram all zero, starts all zero
    origin, h, dims = np.zeros(3, np.float32), np.float32(1.0), np.array([3, 2, 1], np.uint32)
    r = orc.grid_build(np.zeros((0, 8), np.float32), origin, h, dims)
    assert r.conteos.tolist() == [0] * 6 and r.inicios.tolist() == [0] * 7
    assert r.ordenado.size == 0 and r.reordered.shape == (0, 8)
    # one cell: everything lands there, in index order
    parts = np.random.Generator(np.random.PCG64(3)).standard_normal((50, 8)).astype(np.float32)
    r = orc.grid_build(parts, origin, h, np.array([1, 1, 1], np.uint32))
    assert r.conteos.tolist() == [50] and r.inicios.tolist() == [0, 50]
    assert r.ordenado.tolist() == list(range(50))
    # one particle
    r = orc.grid_build(parts[:1], origin, h, dims)
    assert int(r.inicios[-1]) == 1 and r.ordenado.tolist() == [0]


# ---------------------------------------------------------------------------
# Morton (Z-order) cell keys ("Reordenar por celda y la coalescencia de
# memoria", section "El orden de las celdas también importa"). The key is the
# 3-D bit interleave x0 y0 z0 x1 y1 z1 ... (x lowest). Pinned against
# printed-by-hand values of the interleave, against the Z-curve's recursive
# definition (a key is eight times its parent octant's key plus the child
# number x + 2y + 4z), and against the linear numbering it relabels.
# ---------------------------------------------------------------------------


def morton_recursive(kx: int, ky: int, kz: int, bits: int) -> int:
    """Z-curve key by octant recursion (independent of the bit loop)."""
    if bits == 0:
        return 0
    return 8 * morton_recursive(kx >> 1, ky >> 1, kz >> 1, bits - 1) + (kx & 1) + 2 * (ky & 1) + 4 * (kz & 1)


def pin_morton_textbook(orc):
    cases = {
        (0, 0, 0): 0, (1, 0, 0): 1, (0, 1, 0): 2, (0, 0, 1): 4, (1, 1, 1): 7,
        (2, 0, 0): 8, (0, 2, 0): 16, (0, 0, 2): 32, (3, 3, 3): 63, (5, 0, 0): 0b1000001,
        (1023, 0, 0): 0x09249249, (0, 1023, 0): 0x12492492, (0, 0, 1023): 0x24924924,
        (1023, 1023, 1023): (1 << 30) - 1,
    }
    got = orc.morton_keys(list(cases), 10)
    assert got.tolist() == list(cases.values()), got
    assert orc.morton_bits((128, 128, 128)) == 7
    assert orc.morton_bits((16, 16, 16)) == 4
    assert orc.morton_bits((7, 5, 3)) == 3
    assert orc.morton_bits((1, 1, 1)) == 0
    assert orc.morton_bits((1024, 1, 1)) == 10
    for bad in ((1025, 1, 1), (1 << 20, 2, 2)):
        try:
            orc.morton_bits(bad)
        except oracle.OracleError:
            continue
        raise AssertionError(f"morton_bits{bad} should be out of range")


def pin_morton_recursion_bijection(orc):
    """Small grids exhaustively: keys follow the octant recursion and map
    [0, 2^B)^3 one-to-one onto [0, 8^B); aligned runs of 8 keys are 2x2x2 cubes."""
    for bits in range(1, 5):
        side = 1 << bits
        g = np.stack(np.meshgrid(np.arange(side), np.arange(side), np.arange(side), indexing="ij"), -1).reshape(-1, 3)
        got = orc.morton_keys(g, bits).astype(np.int64)
        want = np.array([morton_recursive(int(a), int(b), int(c), bits) for a, b, c in g], dtype=np.int64)
        assert np.array_equal(got, want), bits
        assert np.array_equal(np.sort(got), np.arange(side ** 3))
        inv = np.empty_like(got)
        inv[got] = np.arange(got.size)
        blocks = g[inv].reshape(-1, 8, 3)
        assert np.all(blocks.max(1) - blocks.min(1) == 1) and np.all(blocks.min(1) % 2 == 0)
    rng = np.random.Generator(np.random.PCG64(12))
    g = rng.integers(0, 1024, (500, 3))
    got = orc.morton_keys(g, 10).astype(np.int64)
    assert got.tolist() == [morton_recursive(int(a), int(b), int(c), 10) for a, b, c in g]


def pin_morton_relabels_linear(orc, wl):
    """A Morton build is the linear build with cells renamed: same clamped
    cell per particle, key = interleave of its coordinates, the same counts
    moved to the new keys, zero counts on keys no cell maps to (non-cubic
    grids), and the same stable order within every cell."""
    lin = orc.grid_build(wl.particles, wl.origin, wl.cell_size, wl.dims)
    mor = orc.grid_build(wl.particles, wl.origin, wl.cell_size, wl.dims, morton=True)
    d = [int(v) for v in wl.dims]
    bits = orc.morton_bits(d)
    keys = orc.key_count(wl.origin, wl.cell_size, wl.dims, morton=True)
    assert keys == 1 << (3 * bits)
    c = lin.celdaDe.astype(np.int64)
    xyz = np.stack([c % d[0], (c // d[0]) % d[1], c // (d[0] * d[1])], -1)
    want = np.array([morton_recursive(int(a), int(b), int(e), bits) for a, b, e in xyz], dtype=np.int64)
    assert np.array_equal(mor.celdaDe.astype(np.int64), want)
    cells = np.stack(np.meshgrid(np.arange(d[0]), np.arange(d[1]), np.arange(d[2]), indexing="ij"), -1).reshape(-1, 3)
    lin_of = cells[:, 0] + cells[:, 1] * d[0] + cells[:, 2] * d[0] * d[1]
    key_of = orc.morton_keys(cells, bits).astype(np.int64)
    moved = np.zeros(keys, dtype=np.uint32)
    moved[key_of] = lin.conteos[lin_of]
    assert np.array_equal(mor.conteos, moved)
    check_index_invariants(wl, mor, stable=True, keys=keys)
    for k, lc in zip(key_of[:64], lin_of[:64]):
        a = mor.ordenado[mor.inicios[k]:mor.inicios[k + 1]].tolist()
        b = lin.ordenado[lin.inicios[lc]:lin.inicios[lc + 1]].tolist()
        assert a == b, (k, lc)


# ---------------------------------------------------------------------------
# 27-cell neighbour count (a consumer of the index). Pinned against brute
# force over all pairs (no grid involved), a lattice with a closed-form
# answer (distance exactly equal to the radius counts), and pair symmetry.
# ---------------------------------------------------------------------------


def brute_force_neighbors(particles, radius) -> np.ndarray:
    """#{j != i : (dx*dx + dy*dy) + dz*dz <= r*r}, binary32, all pairs."""
    p = np.ascontiguousarray(particles[:, :3], dtype=np.float32)
    r2 = np.float32(radius) * np.float32(radius)
    out = np.zeros(p.shape[0], dtype=np.int64)
    for s in range(0, p.shape[0], 512):
        d = p[None, :, :] - p[s:s + 512, None, :]  # row i, column j: p[j] - p[i]
        d2 = (d[..., 0] * d[..., 0] + d[..., 1] * d[..., 1]) + d[..., 2] * d[..., 2]
        hit = d2 <= r2
        hit[np.arange(hit.shape[0]), np.arange(s, s + hit.shape[0])] = False  # not itself
        out[s:s + 512] = hit.sum(1)
    return out


def pin_neighbors_brute_force(orc, wl, radius, morton=False):
    """With radius <= cell size and every particle inside the grid, the
    27-cell count equals the all-pairs count."""
    lo = np.asarray(wl.origin, np.float64)
    hi = lo + np.asarray(wl.dims, np.float64) * float(wl.cell_size)
    p = wl.particles[:, :3].astype(np.float64)
    assert np.all((p >= lo) & (p < hi)), "pin needs every particle inside the grid"
    assert radius <= float(wl.cell_size)
    got = orc.neighbor_count(wl.particles, wl.origin, wl.cell_size, wl.dims, radius, morton=morton)
    want = brute_force_neighbors(wl.particles, radius)
    assert np.array_equal(got.astype(np.int64), want), np.nonzero(got != want)[0][:5]
    assert int(got.sum()) % 2 == 0  # every pair counted from both ends


def pin_neighbors_lattice(orc):
    """Particles at the centres of a 6x5x4 grid of unit cells, radius 1: each
    has exactly its axis neighbours (distance 1, equal to the radius; the
    diagonals are at sqrt 2 and sqrt 3), i.e. the sum over axes of
    [k > 0] + [k < dim - 1]. Radius 0.99: none."""
    dims = (6, 5, 4)
    g = np.stack(np.meshgrid(*[np.arange(d) for d in dims], indexing="ij"), -1).reshape(-1, 3)
    rng = np.random.Generator(np.random.PCG64(6))
    g = g[rng.permutation(g.shape[0])]
    parts = np.zeros((g.shape[0], 8), np.float32)
    parts[:, :3] = g + 0.5
    want = sum((g[:, a] > 0).astype(int) + (g[:, a] < dims[a] - 1).astype(int) for a in range(3))
    for morton in (False, True):
        got = orc.neighbor_count(parts, np.zeros(3), 1.0, dims, 1.0, morton=morton)
        assert np.array_equal(got.astype(np.int64), want)
        got = orc.neighbor_count(parts, np.zeros(3), 1.0, dims, 0.99, morton=morton)
        assert not got.any()


def pin_gather_bytes(orc):
    """Byte gather of split state: equals NumPy fancy indexing for every
    element size, with repeated and reversed indices, bit for bit (NaN
    payloads included)."""
    rng = np.random.Generator(np.random.PCG64(44))
    for eb in (4, 8, 12, 16, 20, 32, 48, 64):
        rows = 777
        a = rng.integers(0, 2 ** 32, size=(rows, eb // 4), dtype=np.uint64).astype(np.uint32)
        a[5, 0] = 0x7FC0_0001  # a NaN payload as float32
        for idx in (rng.integers(0, rows, 1000), np.arange(rows)[::-1], np.zeros(3, np.int64)):
            got = orc.gather(a, idx)
            assert np.array_equal(got, a[idx]), eb
    assert orc.gather(np.zeros((4, 8), np.float32), np.zeros(0, np.uint32)).shape == (0, 8)
