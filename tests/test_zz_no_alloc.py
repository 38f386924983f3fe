"""GPU test of ugp_grid_build_noalloc, the build for callers that cannot
allocate: its output against ugp_grid_build's on the same inputs, on two
calls in a row (the second smaller, so the shared fixed workspace holds the
first call's data), in every mode, plus the size limit."""

from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads as W  # noqa: E402
from tests import pins  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ugp():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import uniform_grid_particle_amd as m

    m.load_library()
    return m


def _u32(t):
    return t.detach().cpu().numpy().view(np.uint32)


def _index(r, n):
    return oracle.GridIndex(_u32(r.celdaDe)[:n], _u32(r.conteos), _u32(r.inicios), _u32(r.ordenado)[:n],
                            r.reordered.cpu().numpy()[:n] if r.reordered.numel() else None)


@pytest.mark.parametrize("mode", ["atomic", "stable", "gather", "index_only"])
def test_noalloc_matches_grid_build(ugp, mode):
    dev = torch.device("cuda:0")
    kw = {"stable": mode == "stable", "gather": mode == "gather", "index_only": mode == "index_only"}
    flags = ((ugp.FLAG_STABLE if kw["stable"] else 0) | (ugp.FLAG_GATHER if kw["gather"] else 0)
             | (ugp.FLAG_INDEX_ONLY if kw["index_only"] else 0))
    for wl in (W.make_config("baseline"), W.make_uniform(70_001, 64, seed=41), W.make_config("tiny")):
        print(f"[noalloc] {mode} n={wl.n} dims={wl.dims.tolist()}", flush=True)
        parts = torch.from_numpy(wl.particles).to(dev)
        args = (parts, wl.origin.tolist(), float(wl.cell_size), wl.dims.tolist())
        ref = ugp.grid_build(*args, **kw)
        out, _ = ugp.alloc_outputs(wl.n, wl.dims.tolist(), dev, flags)
        ugp.grid_build_noalloc(*args, out, **kw)
        torch.cuda.synchronize()
        a, b = _index(ref, wl.n), _index(out, wl.n)
        assert np.array_equal(a.celdaDe, b.celdaDe)
        assert np.array_equal(a.conteos, b.conteos)
        assert np.array_equal(a.inicios, b.inicios)
        if kw["index_only"]:  # no records written: every other invariant still holds
            b = oracle.GridIndex(b.celdaDe, b.conteos, b.inicios, b.ordenado, wl.particles[b.ordenado])
        pins.check_index_invariants(wl, b, stable=kw["stable"])
        if kw["stable"]:
            assert np.array_equal(a.ordenado, b.ordenado)
            assert np.array_equal(a.reordered.view(np.uint32), b.reordered.view(np.uint32))
        else:  # the same set in every cell
            ka = np.lexsort((a.ordenado, a.celdaDe[a.ordenado]))
            kb = np.lexsort((b.ordenado, b.celdaDe[b.ordenado]))
            assert np.array_equal(a.ordenado[ka], b.ordenado[kb])


def test_noalloc_rejects_oversized_work(ugp):
    dev = torch.device("cuda:0")
    n, dims = 1_500_000, [128, 128, 128]
    assert ugp.workspace_bytes(n, dims) > ugp.NOALLOC_SCRATCH_BYTES
    parts = torch.zeros((n, 8), dtype=torch.float32, device=dev)
    out, _ = ugp.alloc_outputs(n, dims, dev)
    out.conteos.fill_(-1)
    with pytest.raises(ugp.UGPError) as e:
        ugp.grid_build_noalloc(parts, [0.0, 0.0, 0.0], 1.0, dims, out)
    assert e.value.status == ugp.UGP_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert int(out.conteos[0]) == -1  # nothing was enqueued
