"""GPU parity of the 27-cell neighbour count (ugp_neighbor_count) against
the oracle. Counts are integers decided by binary32 comparisons made in the
same order on both sides, so they must match exactly, in both data orders
(original order through ordenado; the build's reordered records) and both
cell numberings (linear, Morton). Reordered-order counts are checked through
the GPU's own ordenado: counts[k] belongs to particle ordenado[k].
"""

from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from tests import pins  # noqa: E402
from tests.test_parity import _u32  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ugp():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import uniform_grid_particle_amd as m

    m.load_library()
    return m


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def check_neighbors(ugp, orc, wl, radius, morton, stable=False):
    dev = torch.device("cuda:0")
    parts = torch.from_numpy(np.ascontiguousarray(wl.particles)).to(dev)
    args = ([float(v) for v in wl.origin], float(wl.cell_size), [int(v) for v in wl.dims])
    idx = ugp.grid_build(parts, *args, morton=morton, stable=stable)
    ind = ugp.neighbor_count(parts, *args, idx.inicios, idx.ordenado, radius, morton=morton)
    reo = ugp.neighbor_count(idx.reordered, *args, idx.inicios, None, radius, morton=morton)
    torch.cuda.synchronize()
    want = orc.neighbor_count(wl.particles, wl.origin, wl.cell_size, wl.dims, radius, morton=morton)
    got_ind = _u32(ind)
    assert np.array_equal(got_ind, want), f"indirect: {np.count_nonzero(got_ind != want)} differ"
    ordn = _u32(idx.ordenado)
    assert np.array_equal(_u32(reo), want[ordn]), "reordered counts differ"
    return want


@pytest.mark.parametrize("morton", [False, True])
@pytest.mark.parametrize("name", ["tiny", "sparse", "baseline", "contention"])
def test_neighbors_configs(ugp, orc, name, morton):
    print(f"[neighbors] {name} morton={morton}", flush=True)
    wl = W.make_config(name)
    want = check_neighbors(ugp, orc, wl, float(wl.cell_size), morton)
    assert want.sum() % 2 == 0 or name == "contention"  # clamped outsiders break symmetry


@pytest.mark.parametrize("morton", [False, True])
def test_neighbors_sph_like_full_size(ugp, orc, morton):
    """1M particles, 30.5 per cell, ~84 neighbours each (the bench workload)."""
    print(f"[neighbors] sph_like morton={morton}", flush=True)
    wl = W.make_sph_like()
    want = check_neighbors(ugp, orc, wl, W.SPH_RADIUS_FRACTION * float(wl.cell_size), morton)
    assert 70 < want.mean() < 100


def test_neighbors_small_radius_and_stable_index(ugp, orc):
    wl = W.make_config("tiny")
    for frac in (0.0, 0.3, 0.6):
        check_neighbors(ugp, orc, wl, frac * float(wl.cell_size), False, stable=True)


def test_neighbors_noncubic_dense_duplicates(ugp, orc):
    rng = np.random.Generator(np.random.PCG64(17))
    n = 9 * 6 * 4 * 40
    parts = rng.standard_normal((n, 8)).astype(np.float32)
    parts[:, :3] = (rng.random((n, 3)) * np.array([9.0, 6.0, 4.0]) * 0.5 - 1.0).astype(np.float32)
    parts[100:120, :3] = parts[99, :3]
    wl = W.Workload("dense", parts, np.full(3, -1.0, np.float32), np.float32(0.5), np.array([9, 6, 4], np.uint32))
    for morton in (False, True):
        want = check_neighbors(ugp, orc, wl, 0.5, morton)
        assert np.array_equal(want.astype(np.int64), pins.brute_force_neighbors(parts, 0.5))


def test_neighbors_lattice_closed_form(ugp):
    dims = (6, 5, 4)
    g = np.stack(np.meshgrid(*[np.arange(d) for d in dims], indexing="ij"), -1).reshape(-1, 3)
    parts = np.zeros((g.shape[0], 8), np.float32)
    parts[:, :3] = g + 0.5
    want = sum((g[:, a] > 0).astype(int) + (g[:, a] < dims[a] - 1).astype(int) for a in range(3))
    dev = torch.device("cuda:0")
    p = torch.from_numpy(parts).to(dev)
    for morton in (False, True):
        idx = ugp.grid_build(p, [0.0, 0.0, 0.0], 1.0, dims, morton=morton)
        got = ugp.neighbor_count(p, [0.0, 0.0, 0.0], 1.0, dims, idx.inicios, idx.ordenado, 1.0, morton=morton)
        torch.cuda.synchronize()
        assert np.array_equal(_u32(got).astype(np.int64), want)


def test_neighbors_empty_and_errors(ugp):
    dev = torch.device("cuda:0")
    empty = torch.zeros((0, 8), dtype=torch.float32, device=dev)
    idx = ugp.grid_build(empty, [0.0, 0.0, 0.0], 1.0, (4, 4, 4))
    out = ugp.neighbor_count(empty, [0.0, 0.0, 0.0], 1.0, (4, 4, 4), idx.inicios, idx.ordenado, 1.0)
    assert out.numel() == 0
    wl = W.make_config("tiny")
    p = torch.from_numpy(wl.particles).to(dev)
    args = (wl.origin.tolist(), float(wl.cell_size), wl.dims.tolist())
    idx = ugp.grid_build(p, *args)
    for bad in (float("nan"), -1.0, float("inf")):
        with pytest.raises(ugp.UGPError) as e:
            ugp.neighbor_count(p, *args, idx.inicios, idx.ordenado, bad)
        assert e.value.status == ugp.UGP_ERR_ARG
    with pytest.raises(ugp.UGPError) as e:  # counts written over the particles
        ugp.neighbor_count(p, *args, idx.inicios, idx.ordenado, 0.5, out=p.view(torch.int32).reshape(-1))
    assert e.value.status == ugp.UGP_ERR_ALIAS


@pytest.mark.parametrize("seed", range(40))
def test_neighbors_random_sweep(ugp, orc, seed):
    """Seeded random problems: grids of 1-40 cells per axis, up to 40,000
    particles (some outside the domain, some on exact lattice points so that
    distances fall exactly on the radius), radius 0 to one cell, linear or
    Morton keys, atomic or stable index; both data orders against the oracle."""
    rng = np.random.Generator(np.random.PCG64(90_000 + seed))
    dims = [int(v) for v in rng.integers(1, 41, 3)]
    n = int(rng.integers(0, 40_001))
    h = float(np.float32(rng.choice([0.25, 0.1, 1.0 / 3.0, 0.7])))
    origin = (rng.random(3) * 4 - 2).astype(np.float32)
    ext = np.asarray(dims, np.float64) * h
    parts = rng.standard_normal((n, 8)).astype(np.float32)
    parts[:, :3] = (origin + rng.random((n, 3)) * ext * 1.1 - 0.05 * ext).astype(np.float32)
    if n and rng.random() < 0.3:
        k = rng.integers(0, np.asarray(dims) + 1, (n, 3))
        parts[:, :3] = (origin + k * np.float32(h)).astype(np.float32)
    radius = float(np.float32(h * rng.choice([0.0, 0.3, 0.5, 0.87, 1.0])))
    morton = bool(rng.random() < 0.4 and max(dims) <= 32)
    stable = bool(rng.random() < 0.5)
    print(f"[neighbors] seed={seed} n={n} dims={dims} h={h} r={radius} morton={morton}", flush=True)
    wl = W.Workload(f"nb{seed}", parts, origin, np.float32(h), np.asarray(dims, np.uint32))
    check_neighbors(ugp, orc, wl, radius, morton, stable=stable)
