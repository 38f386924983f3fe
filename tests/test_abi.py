"""CPU tests of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments on the host before touching a GPU."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ugp.h")

ugp = pytest.importorskip("uniform_grid_particle_amd")


def _declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ugp_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ugp.library_path()):
        pytest.fail("libugp.so is not built (run __graft_entry__.build())")
    return ugp.load_library()


def test_header_declares_entry_points():
    names = _declared_functions()
    for want in ("ugp_grid_build", "ugp_grid_build_stage", "ugp_grid_workspace_bytes",
                 "ugp_exclusive_scan_u32", "ugp_scan_workspace_bytes", "ugp_reorder",
                 "ugp_status_string", "ugp_abi_version"):
        assert want in names


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(ugp.library_path())
    for name in _declared_functions():
        assert hasattr(raw, name), f"{name} declared in ugp.h but not exported"


def test_status_strings(lib):
    for st in range(0, -8, -1):
        s = ugp.status_string(st)
        assert s and s != "unknown status"
    assert ugp.status_string(-99) == "unknown status"


def test_workspace_sizes(lib):
    a = ugp.workspace_bytes(1_000_000, (128, 128, 128))
    assert a >= 4 * 128 ** 3 and a % 256 == 0
    b = ugp.workspace_bytes(1_000_000, (128, 128, 128), ugp.FLAG_STABLE)
    assert b > a
    assert ugp.workspace_bytes(0, (1, 1, 1)) >= 4
    with pytest.raises(ugp.UGPError) as e:
        ugp.workspace_bytes(10, (0, 4, 4))
    assert e.value.status == ugp.UGP_ERR_RANGE
    with pytest.raises(ugp.UGPError) as e:
        ugp.workspace_bytes(10, ((1 << 24) + 1, 1, 1))
    assert e.value.status == ugp.UGP_ERR_RANGE
    with pytest.raises(ugp.UGPError) as e:
        ugp.workspace_bytes(10, (1 << 16, 1 << 16, 1))
    assert e.value.status == ugp.UGP_ERR_RANGE
    with pytest.raises(ugp.UGPError) as e:
        ugp.workspace_bytes(10, (4, 4, 4), 0x80)
    assert e.value.status == ugp.UGP_ERR_ARG


def _call_build(lib, *, n=4, origin=(0.0, 0.0, 0.0), h=1.0, dims=(4, 4, 4), ptrs=None, ws_bytes=1 << 20,
                flags=0, stage=None):
    """Call ugp_grid_build with fake (never dereferenced) addresses.

    Only argument combinations that fail host validation are used here, so
    nothing is enqueued and no GPU is touched."""
    base = 1 << 40
    p = dict(particles=base, celdaDe=base + (1 << 30), conteos=base + (2 << 30), inicios=base + (3 << 30),
             ordenado=base + (4 << 30), reordered=base + (5 << 30), workspace=base + (6 << 30))
    if ptrs:
        p.update(ptrs)
    o = (ctypes.c_float * 3)(*origin)
    d = (ctypes.c_uint32 * 3)(*dims)
    args = [p["particles"], n, o, ctypes.c_float(h), d, p["celdaDe"], p["conteos"], p["inicios"], p["ordenado"],
            p["reordered"], p["workspace"], ctypes.c_size_t(ws_bytes), flags, None]
    if stage is None:
        return lib.ugp_grid_build(*args)
    return lib.ugp_grid_build_stage(stage, *args)


def test_stage_names(lib):
    assert ugp.stage_names(1000, (128, 128, 128)) == ["chunk_sort", None, None, "tile_sort", None, None]
    # one tile over the whole input: at most 8192 particles and 2^14 keys
    assert ugp.stage_names(4096, (16, 16, 16)) == [None, None, None, "tile_sort", None, None]
    assert ugp.stage_names(8192, (128, 1, 128)) == [None, None, None, "tile_sort", None, None]
    assert ugp.stage_names(8193, (16, 16, 16))[0] == "chunk_sort"
    assert ugp.stage_names(8192, (129, 1, 128))[0] == "chunk_sort"
    assert ugp.stage_names(1, (1, 1, 1), ugp.FLAG_STABLE)[3:5] == ["tile_sort", "stable_sort"]
    assert ugp.stage_names(3_000_000, (128, 128, 128)) == ["coarse_sort", "tile_scan", "rebucket", "tile_sort", None, None]
    assert ugp.stage_names(1000, (128, 128, 128), ugp.FLAG_STABLE)[4:] == ["stable_sort", None]
    assert ugp.stage_names(1000, (128, 128, 128), ugp.FLAG_STABLE | ugp.FLAG_GATHER)[4:] == ["stable_sort", None]
    assert ugp.stage_names(1000, (128, 128, 128), ugp.FLAG_GATHER)[4:] == [None, "gather"]
    assert ugp.stage_names(0, (128, 128, 128)) == ["clear", None, None, None, None, None]
    assert ugp.stage_names(1000, (8192, 8193, 1))[:4] == ["clear", "count", "scan", "scatter"]
    assert ugp.stage_names(1000, (256, 256, 256))[:4] == ["coarse_sort", "tile_scan", "rebucket", "tile_sort"]
    assert ugp.stage_names(1000, (1024, 1024, 64))[:4] == ["coarse_sort", "tile_scan", "rebucket", "tile_sort"]  # 2^26 keys
    assert ugp.stage_names(1000, (1024, 1024, 65))[:4] == ["clear", "count", "scan", "scatter"]


def test_validation_errors_on_host(lib):
    nan, inf = float("nan"), float("inf")
    assert _call_build(lib, h=0.0) == ugp.UGP_ERR_ARG
    assert _call_build(lib, h=-1.0) == ugp.UGP_ERR_ARG
    assert _call_build(lib, h=nan) == ugp.UGP_ERR_ARG
    assert _call_build(lib, h=inf) == ugp.UGP_ERR_ARG
    assert _call_build(lib, h=-0.0) == ugp.UGP_ERR_ARG
    assert _call_build(lib, origin=(0.0, nan, 0.0)) == ugp.UGP_ERR_ARG
    assert _call_build(lib, origin=(inf, 0.0, 0.0)) == ugp.UGP_ERR_ARG
    assert _call_build(lib, dims=(0, 4, 4)) == ugp.UGP_ERR_RANGE
    assert _call_build(lib, dims=(4, (1 << 24) + 1, 4)) == ugp.UGP_ERR_RANGE
    assert _call_build(lib, dims=(1 << 16, 1 << 16, 1)) == ugp.UGP_ERR_RANGE
    assert _call_build(lib, flags=0x100) == ugp.UGP_ERR_ARG
    assert _call_build(lib, ptrs={"conteos": None}) == ugp.UGP_ERR_NULL
    assert _call_build(lib, ptrs={"inicios": None}) == ugp.UGP_ERR_NULL
    assert _call_build(lib, ptrs={"workspace": None}) == ugp.UGP_ERR_NULL
    assert _call_build(lib, ptrs={"particles": None}) == ugp.UGP_ERR_NULL
    assert _call_build(lib, ptrs={"reordered": None}) == ugp.UGP_ERR_NULL
    assert _call_build(lib, ptrs={"conteos": (1 << 40) + (2 << 30) + 4}) == ugp.UGP_ERR_ALIGN
    assert _call_build(lib, ptrs={"particles": (1 << 40) + 8}) == ugp.UGP_ERR_ALIGN
    assert _call_build(lib, ptrs={"workspace": (1 << 40) + (6 << 30) + 16}) == ugp.UGP_ERR_ALIGN
    assert _call_build(lib, ws_bytes=16) == ugp.UGP_ERR_WORKSPACE
    # reordered overlapping particles (double buffer required)
    assert _call_build(lib, ptrs={"reordered": (1 << 40) + 16 * 4}) == ugp.UGP_ERR_ALIAS
    # inicios overlapping conteos
    assert _call_build(lib, ptrs={"inicios": (1 << 40) + (2 << 30) + 64}) == ugp.UGP_ERR_ALIAS
    # unknown stage; timed build without events
    assert _call_build(lib, stage=99) == ugp.UGP_ERR_ARG
    o = (ctypes.c_float * 3)(0, 0, 0)
    d = (ctypes.c_uint32 * 3)(4, 4, 4)
    b = 1 << 40
    assert lib.ugp_grid_build_timed(b, 4, o, ctypes.c_float(1.0), d, b + (1 << 30), b + (2 << 30), b + (3 << 30),
                                    b + (4 << 30), b + (5 << 30), b + (6 << 30), ctypes.c_size_t(1 << 20), 0, None,
                                    0, None, None) == ugp.UGP_ERR_ARG
    assert _call_build(lib, stage=0, h=0.0) == ugp.UGP_ERR_ARG


def test_scan_and_reorder_validation_on_host(lib):
    base = 1 << 40
    need = ctypes.c_size_t(0)
    assert lib.ugp_scan_workspace_bytes(1000, ctypes.byref(need)) == 0 and need.value >= 4
    assert lib.ugp_exclusive_scan_u32(base, 1000, None, base + (1 << 30), need.value, None) == ugp.UGP_ERR_NULL
    assert lib.ugp_exclusive_scan_u32(base, 1000, base + 4, base + (1 << 30), need.value, None) == ugp.UGP_ERR_ALIGN
    assert lib.ugp_exclusive_scan_u32(base, 1000, base + 1024, base + (1 << 30), need.value, None) == ugp.UGP_ERR_ALIAS
    assert lib.ugp_exclusive_scan_u32(base, 1000, base + (1 << 20), base + (1 << 30), 0, None) == ugp.UGP_ERR_WORKSPACE
    assert lib.ugp_reorder(base, 10, base + (1 << 20), 10, base + 64, None) == ugp.UGP_ERR_ALIAS
    assert lib.ugp_reorder(base, 10, None, 10, base + (1 << 21), None) == ugp.UGP_ERR_NULL
    assert lib.ugp_reorder(base + 8, 10, base + (1 << 20), 10, base + (1 << 21), None) == ugp.UGP_ERR_ALIGN
    assert lib.ugp_reorder(None, 0, None, 0, None, None) == ugp.UGP_OK  # n = 0: nothing to do


def test_product_path_has_no_oracle_dependency():
    """The package and the HIP source never reference the oracle."""
    pkg = os.path.join(ROOT, "uniform_grid_particle_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "oracle" not in text.lower(), f"{f} mentions the oracle"
    assert "oracle" not in open(HEADER, encoding="utf-8").read().lower()


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    import importlib

    mod = importlib.import_module("uniform_grid_particle_amd")
    monkeypatch.setattr(mod, "_lib", None)
    monkeypatch.setattr(mod, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        mod.load_library()


def test_diag_validation_on_host(lib):
    """ugp_grid_build_diag / ugp_cell_diag reject bad arguments before any launch."""
    b = 1 << 40
    o = (ctypes.c_float * 3)(0, 0, 0)
    d = (ctypes.c_uint32 * 3)(4, 4, 4)

    def build_diag(diag, h=1.0):
        return lib.ugp_grid_build_diag(b, 4, o, ctypes.c_float(h), d, b + (1 << 30), b + (2 << 30),
                                       b + (3 << 30), b + (4 << 30), b + (5 << 30), b + (6 << 30),
                                       ctypes.c_size_t(1 << 20), 64, diag, 0, None)

    assert build_diag(None) == ugp.UGP_ERR_NULL
    assert build_diag(b + (7 << 30) + 2) == ugp.UGP_ERR_ALIGN
    assert build_diag(b + (2 << 30) + 16) == ugp.UGP_ERR_ALIAS  # inside conteos
    assert build_diag(b + (7 << 30), h=0.0) == ugp.UGP_ERR_ARG
    assert lib.ugp_cell_diag(b, 100, 8, None, None) == ugp.UGP_ERR_NULL
    assert lib.ugp_cell_diag(None, 100, 8, b + (1 << 20), None) == ugp.UGP_ERR_NULL
    assert lib.ugp_cell_diag(b + 4, 100, 8, b + (1 << 20), None) == ugp.UGP_ERR_ALIGN
    assert lib.ugp_cell_diag(b, 100, 8, b + (1 << 20) + 1, None) == ugp.UGP_ERR_ALIGN
    assert lib.ugp_cell_diag(b, 100, 8, b + 396, None) == ugp.UGP_ERR_ALIAS  # last word of conteos
    ev = 1 << 44  # never dereferenced: every case below fails before its launch
    assert lib.ugp_cell_diag_timed(b, 100, 8, b + (1 << 20), None, None, ev) == ugp.UGP_ERR_ARG
    assert lib.ugp_cell_diag_timed(b, 100, 8, b + (1 << 20), None, ev, None) == ugp.UGP_ERR_ARG
    assert lib.ugp_cell_diag_timed(b, 100, 8, None, None, ev, ev) == ugp.UGP_ERR_NULL
    assert lib.ugp_cell_diag_timed(b + 4, 100, 8, b + (1 << 20), None, ev, ev) == ugp.UGP_ERR_ALIGN
    assert lib.ugp_cell_diag_timed(b, 100, 8, b + 396, None, ev, ev) == ugp.UGP_ERR_ALIAS


def test_key_count_on_host(lib):
    assert ugp.key_count((128, 128, 128)) == 128 ** 3
    assert ugp.key_count((7, 5, 3)) == 105
    assert ugp.key_count((128, 128, 128), ugp.FLAG_MORTON) == 128 ** 3
    assert ugp.key_count((7, 5, 3), ugp.FLAG_MORTON) == 512
    assert ugp.key_count((1, 1, 1), ugp.FLAG_MORTON) == 1
    assert ugp.key_count((256, 2, 2), ugp.FLAG_MORTON) == 1 << 24
    assert ugp.key_count((257, 2, 2), ugp.FLAG_MORTON) == 1 << 27
    with pytest.raises(ugp.UGPError) as e:
        ugp.key_count((1025, 1, 1), ugp.FLAG_MORTON)
    assert e.value.status == ugp.UGP_ERR_RANGE
    # the path follows the key count: 7x5x3 Morton has 512 keys (a tile
    # path), 257x2x2 has 2^27 (global-atomic path)
    assert ugp.stage_names(100, (257, 2, 2), ugp.FLAG_MORTON)[0] == "clear"
    assert ugp.stage_names(100, (257, 2, 2))[3] == "tile_sort"
    assert ugp.workspace_bytes(1000, (7, 5, 3), ugp.FLAG_MORTON) > 0


def test_neighbor_validation_on_host(lib):
    b = 1 << 40
    o = (ctypes.c_float * 3)(0, 0, 0)
    d = (ctypes.c_uint32 * 3)(4, 4, 4)

    def call(parts=b, ini=b + (1 << 30), ordn=b + (2 << 30), radius=1.0, counts=b + (3 << 30), flags=0, h=1.0, dims=d):
        return lib.ugp_neighbor_count(parts, 100, o, ctypes.c_float(h), dims, ini, ordn, ctypes.c_float(radius),
                                      counts, flags, None)

    assert call(radius=float("nan")) == ugp.UGP_ERR_ARG
    assert call(radius=-0.5) == ugp.UGP_ERR_ARG
    assert call(h=0.0) == ugp.UGP_ERR_ARG
    assert call(flags=ugp.FLAG_STABLE) == ugp.UGP_ERR_ARG
    assert call(dims=(ctypes.c_uint32 * 3)(0, 4, 4)) == ugp.UGP_ERR_RANGE
    assert call(dims=(ctypes.c_uint32 * 3)(2000, 4, 4), flags=ugp.FLAG_MORTON) == ugp.UGP_ERR_RANGE
    assert call(parts=None) == ugp.UGP_ERR_NULL
    assert call(ini=None) == ugp.UGP_ERR_NULL
    assert call(counts=None) == ugp.UGP_ERR_NULL
    assert call(parts=b + 8) == ugp.UGP_ERR_ALIGN
    assert call(counts=b + (3 << 30) + 2) == ugp.UGP_ERR_ALIGN
    assert call(counts=b + 64) == ugp.UGP_ERR_ALIAS  # inside the particles
    assert call(counts=b + (2 << 30) + 8) == ugp.UGP_ERR_ALIAS  # inside ordenado
    assert lib.ugp_neighbor_count(None, 0, o, ctypes.c_float(1.0), d, None, None, ctypes.c_float(1.0), None, 0,
                                  None) == ugp.UGP_OK  # n = 0: nothing to do


def test_reorder_arrays_validation_on_host(lib):
    b = 1 << 40

    def call(descs, n=100, n_src=100, idx=b):
        arr = (ugp.ArrayDesc * max(1, len(descs)))(*descs)
        return lib.ugp_reorder_arrays(idx, n, n_src, arr, len(descs), None)

    ok = ugp.ArrayDesc(b + (1 << 30), b + (2 << 30), 32)
    assert call([]) == ugp.UGP_ERR_ARG
    assert call([ok] * 9) == ugp.UGP_ERR_ARG
    assert call([ugp.ArrayDesc(b + (1 << 30), b + (2 << 30), 6)]) == ugp.UGP_ERR_ARG
    assert call([ugp.ArrayDesc(b + (1 << 30), b + (2 << 30), 0)]) == ugp.UGP_ERR_ARG
    assert call([ugp.ArrayDesc(b + (1 << 30), b + (2 << 30), 4100)]) == ugp.UGP_ERR_ARG  # > 4096 bytes
    assert call([ugp.ArrayDesc(b + (1 << 30) + 4, b + (2 << 30), 1028)]) == ugp.UGP_ERR_ARG  # > 256 4-byte chunks
    huge = [ugp.ArrayDesc(b + (1 << 30), b + (2 << 30), 1 << 31), ugp.ArrayDesc(b + (3 << 30), b + (4 << 30), (1 << 31) + 4)]
    assert call(huge) == ugp.UGP_ERR_ARG  # sizes whose 32-bit sum would wrap to 4 bytes
    assert call([ugp.ArrayDesc(None, b + (2 << 30), 32)]) == ugp.UGP_ERR_NULL
    assert call([ugp.ArrayDesc(b + (1 << 30) + 2, b + (2 << 30), 32)]) == ugp.UGP_ERR_ALIGN
    assert call([ok], idx=None) == ugp.UGP_ERR_NULL
    assert call([ugp.ArrayDesc(b + (1 << 30), b + (1 << 30) + 64, 32)]) == ugp.UGP_ERR_ALIAS  # dst inside src
    assert call([ok, ugp.ArrayDesc(b + (3 << 30), b + (2 << 30) + 32, 32)]) == ugp.UGP_ERR_ALIAS  # dsts overlap
    assert call([ugp.ArrayDesc(b + (1 << 30), b + 16, 32)]) == ugp.UGP_ERR_ALIAS  # dst over idx
    assert call([ok], n=0, idx=None) == ugp.UGP_OK
