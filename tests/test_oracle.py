"""CPU tests: the oracle against its pins (no GPU needed)."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as W
from tests import pins


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def test_round_f32_helper():
    pins.pin_round_f32_helper()


def test_worked_example_scan(orc):
    pins.pin_worked_example_scan(orc)


def test_worked_example_pipeline(orc):
    pins.pin_worked_example_pipeline(orc)


def test_cell_centres_noncubic(orc):
    pins.pin_cell_centres_noncubic(orc)


def test_special_positions(orc):
    pins.pin_special_positions(orc)


def test_grid_validation(orc):
    pins.pin_grid_validation(orc)


def test_empty_and_degenerate(orc):
    pins.pin_empty_and_degenerate(orc)


def test_diag_closed_form(orc):
    pins.pin_diag_closed_form(orc)


@pytest.mark.parametrize("d", [16, 128])
def test_binary32_model_on_faces(orc, d):
    wl = W.make_boundary_probe((d, d, d), (-5.0, -5.0, -5.0), np.float32(10.0 / d), per_axis_random=512)
    pins.pin_binary32_model(orc, wl)


def test_binary32_model_noncubic_faces(orc):
    wl = W.make_boundary_probe((7, 5, 3), (-1.25, 0.5, 3.0), np.float32(0.3), per_axis_random=256)
    pins.pin_binary32_model(orc, wl)


@pytest.mark.parametrize("h,o,d", [(0.1, -3.0, 64), (0.013, -0.5, 200), (1.0 / 3.0, -2.0, 30)])
def test_binary32_model_nondyadic_faces(orc, h, o, d):
    # Non-binary cell sizes: here a reciprocal multiply or a divide-then-subtract
    # rounding order picks a different cell for some face-adjacent inputs.
    wl = W.make_boundary_probe((d, d, d), (o, o, o), np.float32(h), per_axis_random=512)
    pins.pin_binary32_model(orc, wl)


# Subnormal cell sizes (dyadic 2^-140, non-dyadic 1e-40 and 3e-40): faces
# at subnormal multiples of h, origins at zero and below it.
SUBNORMAL_GRIDS = [(2.0 ** -140, 0.0, 16), (1e-40, 0.0, 16), (3e-40, -2e-39, 12)]


@pytest.mark.parametrize("h,o,d", SUBNORMAL_GRIDS)
def test_binary32_model_subnormal_cell_size(orc, h, o, d):
    wl = W.make_boundary_probe((d, d, d), (o, o, o), np.float32(h), per_axis_random=256)
    assert 0.0 < float(wl.cell_size) < 1.1754944e-38
    pins.pin_binary32_model(orc, wl)
    pins.pin_brute_force_slices(orc, wl)


def test_binary32_model_tiny(orc):
    wl = W.make_config("tiny")
    pins.pin_binary32_model(orc, wl)


def test_exact_floor_tiny(orc):
    pins.pin_exact_floor_far_from_faces(orc, W.make_config("tiny"))


def test_brute_force_tiny(orc):
    pins.pin_brute_force_slices(orc, W.make_config("tiny"))


@pytest.mark.parametrize("name", ["tiny", "sparse", "baseline", "contention"])
def test_library_reductions(orc, name):
    wl = W.make_config(name)
    pins.pin_library_reductions(orc, wl)


def test_contention_workload_shape(orc):
    wl = W.make_config("contention")
    r = orc.grid_build(wl.particles, wl.origin, wl.cell_size, wl.dims)
    assert int(r.conteos.max()) >= 10_000
    hx, hy, hz = wl.meta["hot_cell_xyz"]
    assert int(r.conteos[hx + 128 * hy + 128 * 128 * hz]) >= 10_000
    p = wl.particles[:, :3]
    outside = np.any((p < -5.0) | (p > 5.0), axis=1)
    assert int(outside.sum()) >= 50_000


@pytest.mark.slow
def test_large_invariants(orc):
    wl = W.make_config("large")
    r = orc.grid_build(wl.particles, wl.origin, wl.cell_size, wl.dims)
    pins.check_index_invariants(wl, r, stable=True)
    assert np.array_equal(r.conteos, np.bincount(r.celdaDe, minlength=wl.cells).astype(np.uint32))


def test_workloads_reproducible():
    a = W.make_config("tiny")
    b = W.make_config("tiny")
    assert np.array_equal(a.particles, b.particles)
    c = W.make_config("tiny", seed=2)
    assert not np.array_equal(a.particles, c.particles)
    p = a.particles
    assert p.dtype == np.float32 and p.shape == (4096, 8) and p.flags.c_contiguous
    assert np.all(p[:, :3] >= -5.0) and np.all(p[:, :3] <= 5.0)
    assert np.all((p[:, 3] >= 1.0) & (p[:, 3] <= 4.0))
    assert np.all(p[:, 4:7] == 0.0)
    assert np.all((p[:, 7] >= 0.5) & (p[:, 7] <= 1.5))


# ---------------------------------------------------------------------------
# Mutation test: plant plausible mistakes in a copy of the oracle source and
# check that at least one pin fails for each. This shows the pins can catch
# a dropped term, a wrong sign or index, or a transposed operand.
# ---------------------------------------------------------------------------

MUTATIONS = {
    "axes_transposed": ("c = kx + ky * nx + kz * nxy;", "c = kz + ky * nx + kx * nxy;"),
    "stride_uses_nxy_for_y": ("c = kx + ky * nx + kz * nxy;", "c = kx + ky * nxy + kz * nx;"),
    "sign_flipped": ("float t = p - o;", "float t = o - p;"),
    "reciprocal_multiply": ("float q = t / h;", "float q = t * (1.0f / h);"),
    "divide_then_subtract": (
        "float t = p - o;\n    float q = t / h;",
        "float t = p / h;\n    float q = t - o / h;",
    ),
    "ceil_not_floor": ("float f = floorf(q);", "float f = ceilf(q);"),
    "clamp_off_by_one": ("float top = (float)(dim - 1u);", "float top = (float)(dim);"),
    "inclusive_scan": (
        "inicios[c] = (uint32_t)run;\n        run += conteos[c];",
        "run += conteos[c];\n        inicios[c] = (uint32_t)run;",
    ),
    "histogram_drops_last": (
        "for (uint32_t i = 0; i < n; ++i) {\n        uint32_t c = celdaDe[i];\n        if (c >= cells) return UGPO_ERR_RANGE;\n        conteos[c] += 1u;",
        "for (uint32_t i = 0; i + 1 < n; ++i) {\n        uint32_t c = celdaDe[i];\n        if (c >= cells) return UGPO_ERR_RANGE;\n        conteos[c] += 1u;",
    ),
    "scatter_descending": (
        "for (uint32_t i = 0; i < n; ++i) {\n        uint32_t c = celdaDe[i];\n        if (c >= cells) return UGPO_ERR_RANGE;\n        uint64_t slot",
        "for (uint32_t i = n; i-- > 0;) {\n        uint32_t c = celdaDe[i];\n        if (c >= cells) return UGPO_ERR_RANGE;\n        uint64_t slot",
    ),
    "reorder_scatter_direction": (
        "memcpy(reordered + (size_t)k * 8u, particles + (size_t)src * 8u, 32u);",
        "memcpy(reordered + (size_t)src * 8u, particles + (size_t)k * 8u, 32u);",
    ),
    "reorder_drops_tail": (
        "memcpy(reordered + (size_t)k * 8u, particles + (size_t)src * 8u, 32u);",
        "memcpy(reordered + (size_t)k * 8u, particles + (size_t)src * 8u, 28u);",
    ),
    "diag_counts_cells_not_insertions": (
        "if (v > capacity) ov += (uint64_t)(v - capacity);",
        "if (v > capacity) ov += 1u;",
    ),
    "diag_no_max": ("if (v > mx) mx = v;", "if (v > mx) mx = v - 1;"),
    "morton_axes_swapped": (
        "key |= (uint64_t)((kx >> b) & 1u) << (3u * b);\n        key |= (uint64_t)((ky >> b) & 1u) << (3u * b + 1u);",
        "key |= (uint64_t)((ky >> b) & 1u) << (3u * b);\n        key |= (uint64_t)((kx >> b) & 1u) << (3u * b + 1u);",
    ),
    "morton_stride_off": ("<< (3u * b + 2u);", "<< (3u * b + 3u);"),
    "morton_bits_floor": ("while ((1u << b) < largest) ++b;", "while ((2u << b) <= largest) ++b;"),
    "neighbor_counts_self": ("if (j == i) continue;", "if (j == n) continue;"),
    "neighbor_strict_radius": ("if (d2 <= r2) count += 1u;", "if (d2 < r2) count += 1u;"),
    "neighbor_misses_lower_z": ("for (int64_t z = k[2] - 1; z <= k[2] + 1; ++z) {",
                                "for (int64_t z = k[2]; z <= k[2] + 1; ++z) {"),
    "neighbor_x_window_short": ("for (int64_t x = k[0] - 1; x <= k[0] + 1; ++x) {",
                                "for (int64_t x = k[0] - 1; x <= k[0]; ++x) {"),
    "gather_short_copy": ("memcpy(d + (size_t)k * elem_bytes, s + (size_t)idx[k] * elem_bytes, elem_bytes);",
                          "memcpy(d + (size_t)k * elem_bytes, s + (size_t)idx[k] * elem_bytes, elem_bytes - 4);"),
    "gather_scatter_direction": ("memcpy(d + (size_t)k * elem_bytes, s + (size_t)idx[k] * elem_bytes, elem_bytes);",
                                 "memcpy(d + (size_t)idx[k] * elem_bytes, s + (size_t)k * elem_bytes, elem_bytes);"),
    "morton_drops_top_level": ("for (uint32_t b = 0; b < bits; ++b) {\n        key",
                               "for (uint32_t b = 0; b + 1 < bits; ++b) {\n        key"),
}


def _noncubic_workload():
    """3000 particles on a 7x5x3 grid, some outside it (clamped)."""
    rng = np.random.Generator(np.random.PCG64(33))
    parts = rng.standard_normal((3000, 8)).astype(np.float32)
    parts[:, :3] = (rng.random((3000, 3)) * np.array([8.0, 6.0, 4.0]) - 0.5).astype(np.float32)
    return W.Workload("noncubic", parts, np.zeros(3, np.float32), np.float32(1.0), np.array([7, 5, 3], np.uint32))


def test_morton_textbook(orc):
    pins.pin_morton_textbook(orc)


def test_morton_recursion_bijection(orc):
    pins.pin_morton_recursion_bijection(orc)


@pytest.mark.parametrize("which", ["tiny", "noncubic", "contention_small"])
def test_morton_relabels_linear(orc, which):
    if which == "tiny":
        wl = W.make_config("tiny")
    elif which == "noncubic":
        wl = _noncubic_workload()
    else:  # the contention recipe on a 32^3 grid (hot cell, clusters, clamped outsiders)
        wl = W.make_contention(20_000, 32, seed=4, hot=1000, per_cluster=3000, outside=1000)
    pins.pin_morton_relabels_linear(orc, wl)


def test_gather_bytes(orc):
    pins.pin_gather_bytes(orc)


def test_neighbors_lattice(orc):
    pins.pin_neighbors_lattice(orc)


@pytest.mark.parametrize("morton", [False, True])
@pytest.mark.parametrize("frac", [1.0, 0.6])
def test_neighbors_brute_force(orc, morton, frac):
    wl = W.make_config("tiny")
    pins.pin_neighbors_brute_force(orc, wl, frac * float(wl.cell_size), morton=morton)


def test_neighbors_brute_force_dense_noncubic(orc):
    """~40 particles per cell on a 9x6x4 grid (the pages' 20-60 per cell), duplicates included."""
    rng = np.random.Generator(np.random.PCG64(17))
    n = 9 * 6 * 4 * 40
    parts = rng.standard_normal((n, 8)).astype(np.float32)
    parts[:, :3] = (rng.random((n, 3)) * np.array([9.0, 6.0, 4.0]) * 0.5 - 1.0).astype(np.float32)
    parts[100:120, :3] = parts[99, :3]  # coincident points: distance 0
    wl = W.Workload("dense", parts, np.full(3, -1.0, np.float32), np.float32(0.5), np.array([9, 6, 4], np.uint32))
    for morton in (False, True):
        pins.pin_neighbors_brute_force(orc, wl, 0.5, morton=morton)


def _all_pins(orc_m):
    tiny = W.make_config("tiny")
    face16 = W.make_boundary_probe((16, 16, 16), (-5.0, -5.0, -5.0), np.float32(0.625), per_axis_random=128)
    face128 = W.make_boundary_probe((128, 128, 128), (-5.0, -5.0, -5.0), np.float32(0.078125), per_axis_random=128)
    face_nd = W.make_boundary_probe((64, 64, 64), (-3.0, -3.0, -3.0), np.float32(0.1), per_axis_random=128)
    noncubic = _noncubic_workload()
    checks = [
        lambda: pins.pin_worked_example_scan(orc_m),
        lambda: pins.pin_worked_example_pipeline(orc_m),
        lambda: pins.pin_cell_centres_noncubic(orc_m),
        lambda: pins.pin_special_positions(orc_m),
        lambda: pins.pin_empty_and_degenerate(orc_m),
        lambda: pins.pin_diag_closed_form(orc_m),
        lambda: pins.pin_binary32_model(orc_m, face16),
        lambda: pins.pin_binary32_model(orc_m, face128),
        lambda: pins.pin_binary32_model(orc_m, face_nd),
        lambda: pins.pin_library_reductions(orc_m, tiny),
        lambda: pins.pin_morton_textbook(orc_m),
        lambda: pins.pin_morton_recursion_bijection(orc_m),
        lambda: pins.pin_morton_relabels_linear(orc_m, tiny),
        lambda: pins.pin_morton_relabels_linear(orc_m, noncubic),
        lambda: pins.pin_neighbors_lattice(orc_m),
        lambda: pins.pin_gather_bytes(orc_m),
        lambda: pins.pin_neighbors_brute_force(orc_m, tiny, float(tiny.cell_size)),
    ]
    failed = 0
    for chk in checks:
        try:
            chk()
        except (AssertionError, oracle.OracleError):
            failed += 1
    return failed


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(mutation, tmp_path):
    src = open(oracle._SRC, encoding="utf-8").read()
    old, new = MUTATIONS[mutation]
    assert src.count(old) >= 1, f"mutation anchor missing from oracle source: {old!r}"
    mutated = src.replace(old, new)
    path = tmp_path / "mut.c"
    path.write_text(mutated, encoding="utf-8")
    lib = oracle.build(str(path), str(tmp_path / f"libmut_{mutation}.so"))
    orc_m = oracle.Oracle(lib)
    assert _all_pins(orc_m) >= 1, f"no pin caught the planted mistake {mutation}"


def test_unmutated_oracle_passes_all_pins(orc):
    assert _all_pins(orc) == 0
