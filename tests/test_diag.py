"""GPU parity of the overflow diagnostics (page "Contar partículas por
celda", section "Detectar el desbordamiento sin salir de la GPU").

Expected values come from the oracle's closed form over its own histogram
(largest count; sum of max(0, count - capacity)), which the CPU tests pin
against a replay of the per-insertion rule. Every build here also checks
the index itself against the oracle, so the diagnostic variant of each
kernel is held to the same bar as the plain one.
"""

from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from tests.test_parity import MODES, _u32, assert_parity  # noqa: E402

pytestmark = pytest.mark.gpu

CAPS = (0, 1, 3, 20, 64, 10_000, 0xFFFFFFFF)


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


def run_diag(ugp, wl, capacity, mode="atomic"):
    dev = torch.device("cuda:0")
    parts = torch.from_numpy(np.ascontiguousarray(wl.particles)).to(dev)
    diag = torch.full((2,), -1, dtype=torch.int32, device=dev)  # stale content must be overwritten
    r, _ = ugp.grid_build_diag(parts, [float(v) for v in wl.origin], float(wl.cell_size),
                               [int(v) for v in wl.dims], capacity, diag=diag, **MODES[mode])
    torch.cuda.synchronize()
    got = oracle.GridIndex(_u32(r.celdaDe)[: wl.n], _u32(r.conteos), _u32(r.inicios),
                           _u32(r.ordenado)[: wl.n], r.reordered.cpu().numpy()[: wl.n])
    return got, tuple(int(v) for v in _u32(diag))


@pytest.mark.parametrize("name", ["tiny", "sparse", "baseline", "contention"])
def test_diag_configs(ugp, orc, name):
    print(f"[diag] {name}", flush=True)
    wl = W.make_config(name)
    ref = orc.grid_build(wl.particles, wl.origin, wl.cell_size, wl.dims)
    for i, cap in enumerate(CAPS):
        mode = list(MODES)[i % len(MODES)]
        got, d = run_diag(ugp, wl, cap, mode)
        assert_parity(wl, got, ref, mode)
        assert d == orc.diag(ref.conteos, cap), f"{name} cap={cap} mode={mode}"
    if name == "contention":  # the hot cell holds at least 10,000 particles
        assert orc.diag(ref.conteos, 64)[0] >= 10_000


def test_diag_large_tiled_path(ugp, orc):
    """16,777,216 particles on 256^3: the bucketed path (diagnostics folded into its tile kernel)."""
    print("[diag] large", flush=True)
    wl = W.make_config("large")
    assert ugp.stage_names(wl.n, wl.dims.tolist())[0] == "coarse_sort"
    ref = orc.grid_build(wl.particles, wl.origin, wl.cell_size, wl.dims)
    got, d = run_diag(ugp, wl, 3)
    assert_parity(wl, got, ref, "atomic")
    assert d == orc.diag(ref.conteos, 3)


def test_diag_direct_path(ugp, orc):
    """More than 2^26 cells (global-atomic path) with one dense cell."""
    dims = (8192, 8193, 1)
    n = 100_003
    rng = np.random.Generator(np.random.PCG64(77))
    parts = rng.standard_normal((n, 8)).astype(np.float32)
    parts[:, 0] = (rng.random(n) * 8192).astype(np.float32)
    parts[:, 1] = (rng.random(n) * 8193).astype(np.float32)
    parts[:, 2] = 0.5
    parts[: n // 7, :3] = parts[0, :3]
    wl = W.Workload("direct", parts, np.zeros(3, np.float32), np.float32(1.0), np.asarray(dims, np.uint32))
    assert ugp.stage_names(n, dims)[0] == "clear"
    ref = orc.grid_build(wl.particles, wl.origin, wl.cell_size, wl.dims)
    for cap in (0, 2, n):
        got, d = run_diag(ugp, wl, cap)
        assert_parity(wl, got, ref, "atomic")
        assert d == orc.diag(ref.conteos, cap)


@pytest.mark.parametrize("n", [0, 1, 5000, 16385, 40000])
def test_diag_one_cell_and_empty(ugp, orc, n):
    """All particles in one cell (oversized tile above 8192 particles) and n == 0."""
    rng = np.random.Generator(np.random.PCG64(1000 + n))
    parts = rng.standard_normal((n, 8)).astype(np.float32)
    wl = W.Workload("one_cell", parts, np.zeros(3, np.float32), np.float32(1.0), np.array([1, 1, 1], np.uint32))
    ref = orc.grid_build(wl.particles, wl.origin, wl.cell_size, wl.dims)
    for cap in (0, 7, n, n + 1):
        got, d = run_diag(ugp, wl, cap)
        assert d == orc.diag(ref.conteos, cap) == (n, max(0, n - cap))
        if n:
            assert_parity(wl, got, ref, "atomic")


@pytest.mark.parametrize("cells", [0, 1, 3, 4, 5, 4099, (1 << 20) + 7, 2_097_152])
def test_cell_diag_entry_point(ugp, orc, cells):
    """ugp_cell_diag over synthetic histograms of ragged lengths."""
    rng = np.random.Generator(np.random.PCG64(cells))
    counts = rng.poisson(0.5, cells).astype(np.uint32)
    if cells:
        counts[rng.integers(0, cells, size=min(cells, 5))] = rng.integers(0, 70_000, size=min(cells, 5))
    dev = torch.device("cuda:0")
    t = torch.from_numpy(counts.view(np.int32)).to(dev)
    out = torch.full((2,), -1, dtype=torch.int32, device=dev)
    for cap in (0, 1, 64, 0xFFFFFFFF):
        ugp.cell_diag(t, cap, out=out)
        torch.cuda.synchronize()
        assert tuple(int(v) for v in _u32(out)) == orc.diag(counts, cap), f"cells={cells} cap={cap}"
    # the timed entry point runs the same kernel and records its own events
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out.fill_(-1)
    ugp.cell_diag_timed(t, 64, e0, e1, out=out)
    torch.cuda.synchronize()
    assert tuple(int(v) for v in _u32(out)) == orc.diag(counts, 64), f"timed cells={cells}"
    assert e0.elapsed_time(e1) >= 0.0
