"""GPU parity over seeded sweeps of random problems.

Each case draws a grid (1 to 80 cells per axis, some axes of one cell), a
particle count (0 to 120,000), a position mix (uniform, a few dense clumps,
points outside the domain, exact cell faces) and a flag set (stable, gather,
index only, Morton keys, overflow diagnostics), so that the single-tile,
staged, oversized-tile and fix-up code paths are all crossed many times.
Every case is checked against the oracle by the rules of test_parity.py:
celdaDe, conteos, inicios and the diagnostics bit-exact; ordenado element
for element in stable mode, otherwise per cell; reordered bit-exact against
the GPU's own ordenado (or the oracle's, in stable mode).

A second, shorter sweep draws larger problems (120,000 to 3,000,000
particles on grids of up to 300 cells per axis), which reach the staged
path's limits, the bucketed path and large tiles past the staged capacity;
a third draws problems past 2^26 keys, for the global-atomic path.
"""

from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from tests import pins  # noqa: E402
import workloads as W  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = 160


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


def _u32(t):
    return t.detach().cpu().numpy().view(np.uint32)


def draw_case(seed: int):
    rng = np.random.Generator(np.random.PCG64(1000 + seed))
    dims = [int(v) for v in rng.integers(1, 81, 3)]
    for a in range(3):
        if rng.random() < 0.15:
            dims[a] = 1
    n = int(rng.choice([0, 1, 2, 17, int(rng.integers(1, 9000)), int(rng.integers(9000, 30001)),
                        int(rng.integers(30001, 120001))],
                       p=[0.03, 0.04, 0.04, 0.05, 0.39, 0.35, 0.10]))
    h = np.float32(rng.choice([0.25, 0.1, 1.0 / 3.0, 0.7]))
    origin = (rng.random(3) * 4 - 2).astype(np.float32)
    ext = np.asarray(dims, np.float64) * float(h)
    parts = rng.standard_normal((n, 8)).astype(np.float32)
    parts[:, :3] = (origin + rng.random((n, 3)) * ext).astype(np.float32)
    if n:
        kind = rng.integers(0, 4)
        if kind == 1:  # a few dense clumps
            for _ in range(int(rng.integers(1, 4))):
                m = rng.random(n) < rng.uniform(0.05, 0.4)
                centre = origin + rng.random(3) * ext
                parts[m, :3] = (centre + rng.standard_normal((int(m.sum()), 3)) * float(h) * 0.3).astype(np.float32)
        elif kind == 2:  # points outside the domain on every side
            m = rng.random(n) < 0.2
            parts[m, :3] = (origin + (rng.random((int(m.sum()), 3)) * 1.6 - 0.3) * ext).astype(np.float32)
        elif kind == 3:  # exact cell faces
            m = rng.random(n) < 0.3
            k = rng.integers(0, np.asarray(dims) + 1, (int(m.sum()), 3))
            parts[m, :3] = (origin + k * h).astype(np.float32)
    flags = dict(stable=bool(rng.random() < 0.45), gather=bool(rng.random() < 0.25),
                 index_only=bool(rng.random() < 0.15),
                 morton=bool(rng.random() < 0.3 and max(dims) <= 64))
    cap = int(rng.integers(0, 40)) if rng.random() < 0.35 else None
    wl = W.Workload(f"sweep{seed}", parts, origin, h, np.asarray(dims, np.uint32))
    return wl, flags, cap


LARGE_CASES = 12


def draw_large_case(seed: int):
    rng = np.random.Generator(np.random.PCG64(50_000 + seed))
    dims = [int(v) for v in rng.integers(1, 301, 3)]
    for a in range(3):
        if rng.random() < 0.1:
            dims[a] = 1
    n = int(rng.integers(120_000, 3_000_001))
    h = np.float32(rng.choice([0.25, 0.5, 1.0 / 3.0]))
    origin = (rng.random(3) * 4 - 2).astype(np.float32)
    ext = np.asarray(dims, np.float64) * float(h)
    parts = rng.standard_normal((n, 8)).astype(np.float32)
    parts[:, :3] = (origin + rng.random((n, 3)) * ext).astype(np.float32)
    kind = rng.integers(0, 3)
    if kind == 1:  # dense clumps of varying width
        for _ in range(int(rng.integers(1, 4))):
            m = rng.random(n) < rng.uniform(0.02, 0.3)
            centre = origin + rng.random(3) * ext
            width = float(h) * rng.uniform(0.1, 3.0)
            parts[m, :3] = (centre + rng.standard_normal((int(m.sum()), 3)) * width).astype(np.float32)
    elif kind == 2:  # points outside the domain on every side
        m = rng.random(n) < 0.2
        parts[m, :3] = (origin + (rng.random((int(m.sum()), 3)) * 1.6 - 0.3) * ext).astype(np.float32)
    flags = dict(stable=bool(rng.random() < 0.45), gather=bool(rng.random() < 0.2),
                 index_only=bool(rng.random() < 0.1),
                 morton=bool(rng.random() < 0.25 and max(dims) <= 256))
    cap = int(rng.integers(0, 60)) if rng.random() < 0.25 else None
    wl = W.Workload(f"large_sweep{seed}", parts, origin, h, np.asarray(dims, np.uint32))
    return wl, flags, cap


DIRECT_CASES = 4


def draw_direct_case(seed: int):
    """Past 2^26 keys (the global-atomic path): a wide flat linear grid, or
    Morton keys on a grid wider than 256 cells (padded to 2^27 keys)."""
    rng = np.random.Generator(np.random.PCG64(80_000 + seed))
    if seed % 2 == 0:
        dims = [int(rng.integers(8200, 9000)), int(rng.integers(8193, 9000)), 1]
        morton = False
    else:
        dims = [int(v) for v in rng.integers(257, 513, 3)]
        dims[int(rng.integers(0, 3))] = int(rng.integers(1, 40))
        morton = True
    n = int(rng.integers(1, 400_001))
    ext = np.asarray(dims, np.float64)
    parts = rng.standard_normal((n, 8)).astype(np.float32)
    parts[:, :3] = (rng.random((n, 3)) * ext * 1.02 - 0.01 * ext).astype(np.float32)
    if rng.random() < 0.5:
        m = rng.random(n) < rng.uniform(0.01, 0.2)
        parts[m, :3] = parts[0, :3]  # one dense cell
    flags = dict(stable=bool(rng.random() < 0.5), gather=bool(rng.random() < 0.3),
                 index_only=bool(rng.random() < 0.1), morton=morton)
    cap = int(rng.integers(0, 40)) if rng.random() < 0.3 else None
    wl = W.Workload(f"direct_sweep{seed}", parts, np.zeros(3, np.float32), np.float32(1.0),
                    np.asarray(dims, np.uint32))
    return wl, flags, cap


@pytest.mark.parametrize("seed", range(CASES))
def test_random_case(ugp, orc, seed):
    check_case(ugp, orc, *draw_case(seed), seed)


@pytest.mark.parametrize("seed", range(LARGE_CASES))
def test_random_large_case(ugp, orc, seed):
    check_case(ugp, orc, *draw_large_case(seed), seed)


@pytest.mark.parametrize("seed", range(DIRECT_CASES))
def test_random_direct_case(ugp, orc, seed):
    wl, flags, cap = draw_direct_case(seed)
    fl = ugp.FLAG_MORTON if flags["morton"] else 0
    assert ugp.stage_names(wl.n, wl.dims.tolist(), fl)[:4] == ["clear", "count", "scan", "scatter"]
    check_case(ugp, orc, wl, flags, cap, seed)


def check_case(ugp, orc, wl, flags, cap, seed):
    print(f"[sweep] seed={seed} n={wl.n} dims={wl.dims.tolist()} flags={flags} cap={cap}", flush=True)
    ref = orc.grid_build(wl.particles, wl.origin, wl.cell_size, wl.dims, morton=flags["morton"])
    dev = torch.device("cuda:0")
    parts = torch.from_numpy(np.ascontiguousarray(wl.particles)).to(dev)
    args = ([float(v) for v in wl.origin], float(wl.cell_size), [int(v) for v in wl.dims])
    if cap is None:
        r = ugp.grid_build(parts, *args, **flags)
        diag = None
    else:
        r, diag = ugp.grid_build_diag(parts, *args, cap, stable=flags["stable"], gather=flags["gather"],
                                      morton=flags["morton"])
    torch.cuda.synchronize()
    n = wl.n
    celdaDe, conteos, inicios = _u32(r.celdaDe)[:n], _u32(r.conteos), _u32(r.inicios)
    ordenado = _u32(r.ordenado)[:n]
    assert np.array_equal(celdaDe, ref.celdaDe)
    assert np.array_equal(conteos, ref.conteos)
    assert np.array_equal(inicios, ref.inicios)
    if flags["stable"]:
        assert np.array_equal(ordenado, ref.ordenado)
    elif n:
        c = ref.celdaDe[ordenado].astype(np.int64)
        key = np.lexsort((ordenado, c))
        assert np.array_equal(ordenado[key], ref.ordenado)
    if diag is not None:
        assert _u32(diag).tolist() == list(orc.diag(ref.conteos, cap))
    records = cap is not None or not flags["index_only"]
    rec = r.reordered.cpu().numpy()[:n] if records else wl.particles[ordenado]
    if records:
        assert np.array_equal(rec.view(np.uint32), wl.particles.view(np.uint32)[ordenado])
    pins.check_index_invariants(wl, oracle.GridIndex(celdaDe, conteos, inicios, ordenado, rec),
                                stable=flags["stable"], keys=conteos.size if flags["morton"] else None)
