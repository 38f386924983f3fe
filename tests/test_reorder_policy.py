"""GPU tests of the reorder policies of page "Reordenar por celda y la
coalescencia de memoria": several arrays gathered with one index in one
kernel (section "El kernel de reordenación"; hot/cold split of page "El
estado de las partículas en storage buffers"), and the index-only build used
to reorder every few frames (section "Reordenar o no").

Gathers are compared byte for byte with the oracle's gather; index-only
builds with the oracle's index; the neighbour count through ordenado on an
array reordered some frames ago with the oracle's count on the same data.
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

DEV = "cuda:0"


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


def _arrays(rng, n, shapes):
    out = []
    for shp, dt in shapes:
        a = rng.integers(0, 2 ** 32, size=(n,) + shp, dtype=np.uint64).astype(np.uint32).view(dt)
        out.append(np.ascontiguousarray(a))
    return out


@pytest.mark.parametrize("shapes", [
    [((8,), np.float32), ((8,), np.float32)],                     # hot kinematics + cold appearance (16-byte chunks)
    [((8,), np.float32), ((8,), np.float32), ((), np.uint32)],    # plus a colour word (4-byte chunks)
    [((3,), np.float32)],                                         # 12-byte elements
    [((16,), np.float32), ((4,), np.int32), ((2,), np.float32), ((), np.float32), ((5,), np.uint32)],
    [((64,), np.float32)] * 4,                                    # 1 KiB per element, 16-byte chunks
])
@pytest.mark.parametrize("n", [1, 3, 1000, 250_003])
def test_reorder_arrays_matches_oracle(ugp, orc, shapes, n):
    rng = np.random.Generator(np.random.PCG64(n + len(shapes)))
    n_src = n + 17
    srcs = _arrays(rng, n_src, shapes)
    idx = rng.integers(0, n_src, n).astype(np.uint32)
    idx[: min(n, 5)] = n_src - 1  # repeated and last entries
    outs = ugp.reorder_arrays(torch.from_numpy(idx.view(np.int32)).to(DEV), [torch.from_numpy(a).to(DEV) for a in srcs])
    torch.cuda.synchronize()
    for a, o in zip(srcs, outs):
        assert np.array_equal(o.cpu().numpy().view(np.uint32), orc.gather(a, idx).view(np.uint32))


def test_reorder_arrays_with_build_index_and_skips(ugp, orc):
    """The build's ordenado as the index; out-of-range entries leave the
    destination untouched."""
    wl = W.make_config("baseline")
    dev = torch.device(DEV)
    parts = torch.from_numpy(wl.particles).to(dev)
    idx = ugp.grid_build(parts, wl.origin.tolist(), float(wl.cell_size), wl.dims.tolist(), index_only=True)
    rng = np.random.Generator(np.random.PCG64(9))
    cold = _arrays(rng, wl.n, [((8,), np.float32)])[0]
    hot_out, cold_out = ugp.reorder_arrays(idx.ordenado, [parts, torch.from_numpy(cold).to(dev)])
    torch.cuda.synchronize()
    ordn = _u32(idx.ordenado)
    assert np.array_equal(hot_out.cpu().numpy().view(np.uint32), orc.gather(wl.particles, ordn).view(np.uint32))
    assert np.array_equal(cold_out.cpu().numpy().view(np.uint32), orc.gather(cold, ordn).view(np.uint32))
    bad = ordn.copy()
    bad[::7] = wl.n + 5
    sentinel = torch.full((wl.n, 8), -7.0, device=dev)
    ugp.reorder_arrays(torch.from_numpy(bad.view(np.int32)).to(dev), [parts], outs=[sentinel])
    torch.cuda.synchronize()
    got = sentinel.cpu().numpy()
    ok = bad < wl.n
    assert np.array_equal(got[ok].view(np.uint32), wl.particles[bad[ok]].view(np.uint32))
    assert np.all(got[~ok] == -7.0)


def test_reorder_arrays_errors(ugp):
    dev = torch.device(DEV)
    idx = torch.zeros(10, dtype=torch.int32, device=dev)
    a = torch.zeros((10, 8), device=dev)
    with pytest.raises(ugp.UGPError) as e:
        ugp.reorder_arrays(idx, [a] * 9)
    assert e.value.status == ugp.UGP_ERR_ARG
    with pytest.raises(ugp.UGPError) as e:
        ugp.reorder_arrays(idx, [a], outs=[a])  # writes over its own source
    assert e.value.status == ugp.UGP_ERR_ALIAS
    with pytest.raises(ugp.UGPError) as e:
        ugp.reorder_arrays(idx, [torch.zeros((10, 3), dtype=torch.int16, device=dev)])  # 6-byte elements
    assert e.value.status == ugp.UGP_ERR_ARG


@pytest.mark.parametrize("name,flags", [("tiny", ()), ("baseline", ()), ("contention", ("stable",)),
                                        ("baseline", ("morton",)), ("sparse", ("stable", "morton"))])
def test_index_only_build(ugp, orc, name, flags):
    wl = W.make_config(name)
    morton = "morton" in flags
    stable = "stable" in flags
    dev = torch.device(DEV)
    parts = torch.from_numpy(wl.particles).to(dev)
    r = ugp.grid_build(parts, wl.origin.tolist(), float(wl.cell_size), wl.dims.tolist(), index_only=True,
                       morton=morton, stable=stable)
    torch.cuda.synchronize()
    ref = orc.grid_build(wl.particles, wl.origin, wl.cell_size, wl.dims, morton=morton)
    assert np.array_equal(_u32(r.celdaDe), ref.celdaDe)
    assert np.array_equal(_u32(r.conteos), ref.conteos)
    assert np.array_equal(_u32(r.inicios), ref.inicios)
    ordn = _u32(r.ordenado)
    if stable:
        assert np.array_equal(ordn, ref.ordenado)
    else:
        c = ref.celdaDe[ordn].astype(np.int64)
        assert np.array_equal(ordn[np.lexsort((ordn, c))], ref.ordenado)
    assert r.reordered.numel() == 0


def test_index_only_other_paths(ugp, orc):
    """Bucketed path (3M particles on 256^3) and global-atomic path (> 2^26 cells)."""
    dev = torch.device(DEV)
    for wl in (W.make_uniform(3_000_000, 256, seed=61),
               W.Workload("direct", np.random.Generator(np.random.PCG64(3)).random((50_000, 8)).astype(np.float32) * 4000,
                          np.zeros(3, np.float32), np.float32(1.0), np.array([8192, 8193, 1], np.uint32))):
        r = ugp.grid_build(torch.from_numpy(wl.particles).to(dev), wl.origin.tolist(), float(wl.cell_size),
                           wl.dims.tolist(), index_only=True)
        torch.cuda.synchronize()
        ref = orc.grid_build(wl.particles, wl.origin, wl.cell_size, wl.dims)
        assert np.array_equal(_u32(r.inicios), ref.inicios)
        ordn = _u32(r.ordenado)
        c = ref.celdaDe[ordn].astype(np.int64)
        assert np.array_equal(ordn[np.lexsort((ordn, c))], ref.ordenado)


def test_reorder_every_few_frames(ugp, orc):
    """Frame 0 builds and reorders; the next frames move the particles a
    little, rebuild the index only, and query neighbours through ordenado on
    the array reordered at frame 0. Counts equal the oracle's on the moved
    data every frame."""
    wl = W.make_sph_like(n=200_000, d=20)
    dev = torch.device(DEV)
    args = (wl.origin.tolist(), float(wl.cell_size), wl.dims.tolist())
    radius = W.SPH_RADIUS_FRACTION * float(wl.cell_size)
    idx0 = ugp.grid_build(torch.from_numpy(wl.particles).to(dev), *args)
    state = idx0.reordered.clone()
    rng = np.random.Generator(np.random.PCG64(5))
    for frame in range(1, 4):
        host = state.cpu().numpy()
        host[:, :3] += (rng.standard_normal((wl.n, 3)) * 0.05 * float(wl.cell_size)).astype(np.float32)
        state = torch.from_numpy(host).to(dev)
        r = ugp.grid_build(state, *args, index_only=True)
        counts = ugp.neighbor_count(state, *args, r.inicios, r.ordenado, radius)
        torch.cuda.synchronize()
        want = orc.neighbor_count(host, wl.origin, wl.cell_size, wl.dims, radius)
        assert np.array_equal(_u32(counts), want), frame
        # the array reordered at frame 0 is still nearly in cell order
        moved = np.abs(_u32(r.ordenado).astype(np.int64) - np.arange(wl.n))
        assert np.median(moved) < 0.01 * wl.n
