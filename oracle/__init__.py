"""CPU oracle for the uniform-grid index build -- TEST INFRASTRUCTURE ONLY.

Plain, sequential C (``ugp_oracle.c``) behind ctypes. Only the tests, the
smoke check and the benchmark's CPU-baseline leg may import this package;
the GPU library never does, and this package imports nothing from it.

Every function returns NumPy arrays computed on the host. See the C file's
header for which page and section each step follows.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ugp_oracle.c")
_LIB = os.path.join(_HERE, "libugp_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared"]

_u32p = ctypes.POINTER(ctypes.c_uint32)

ORDER_LINEAR = 0  # cell numbering x + y*nx + z*nx*ny
ORDER_MORTON = 1  # Z-order bit interleave
_f32p = ctypes.POINTER(ctypes.c_float)


def build(src: str = _SRC, out: str = _LIB, extra: list[str] | None = None) -> str:
    """Compile the oracle with gcc; returns the path of the shared library."""
    cmd = ["gcc", *CFLAGS, *(extra or []), src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class OracleError(RuntimeError):
    pass


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        self.path = path
        self._lib = lib
        lib.ugp_oracle_check_grid.argtypes = [_f32p, ctypes.c_float, _u32p, ctypes.POINTER(ctypes.c_uint64)]
        lib.ugp_oracle_cell_index.argtypes = [_f32p, ctypes.c_uint32, _f32p, ctypes.c_float, _u32p, _u32p]
        lib.ugp_oracle_histogram.argtypes = [_u32p, ctypes.c_uint32, ctypes.c_uint32, _u32p]
        lib.ugp_oracle_exclusive_scan.argtypes = [_u32p, ctypes.c_uint32, _u32p]
        lib.ugp_oracle_scatter.argtypes = [_u32p, ctypes.c_uint32, _u32p, ctypes.c_uint32, _u32p, _u32p]
        lib.ugp_oracle_reorder.argtypes = [_f32p, _u32p, ctypes.c_uint32, _f32p]
        lib.ugp_oracle_grid_build.argtypes = [
            _f32p, ctypes.c_uint32, _f32p, ctypes.c_float, _u32p,
            _u32p, _u32p, _u32p, _u32p, _f32p, _u32p,
        ]
        lib.ugp_oracle_morton_bits.argtypes = [_u32p, ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint64)]
        lib.ugp_oracle_morton_key.argtypes = [ctypes.c_uint32] * 4
        lib.ugp_oracle_morton_key.restype = ctypes.c_uint32
        lib.ugp_oracle_morton_keys.argtypes = [_u32p, ctypes.c_uint32, ctypes.c_uint32, _u32p]
        lib.ugp_oracle_key_count.argtypes = [_f32p, ctypes.c_float, _u32p, ctypes.c_uint32,
                                             ctypes.POINTER(ctypes.c_uint64)]
        lib.ugp_oracle_cell_key.argtypes = [_f32p, ctypes.c_uint32, _f32p, ctypes.c_float, _u32p,
                                            ctypes.c_uint32, _u32p]
        lib.ugp_oracle_grid_build_keyed.argtypes = [
            _f32p, ctypes.c_uint32, _f32p, ctypes.c_float, _u32p, ctypes.c_uint32,
            _u32p, _u32p, _u32p, _u32p, _f32p, _u32p,
        ]
        lib.ugp_oracle_neighbor_count.argtypes = [
            _f32p, ctypes.c_uint32, _f32p, ctypes.c_float, _u32p, ctypes.c_uint32,
            _u32p, _u32p, ctypes.c_float, _u32p,
        ]
        lib.ugp_oracle_gather_bytes.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32, _u32p,
                                                 ctypes.c_uint32, ctypes.c_void_p]
        lib.ugp_oracle_diag.argtypes = [
            _u32p, ctypes.c_uint32, ctypes.c_uint32,
            ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint32),
        ]
        for fn in (
            lib.ugp_oracle_check_grid, lib.ugp_oracle_cell_index, lib.ugp_oracle_histogram,
            lib.ugp_oracle_exclusive_scan, lib.ugp_oracle_scatter, lib.ugp_oracle_reorder,
            lib.ugp_oracle_grid_build, lib.ugp_oracle_diag, lib.ugp_oracle_morton_bits,
            lib.ugp_oracle_morton_keys, lib.ugp_oracle_key_count, lib.ugp_oracle_cell_key,
            lib.ugp_oracle_grid_build_keyed, lib.ugp_oracle_neighbor_count, lib.ugp_oracle_gather_bytes,
        ):
            fn.restype = ctypes.c_int

    # -- helpers -------------------------------------------------------
    @staticmethod
    def _p(a: np.ndarray, t):
        return a.ctypes.data_as(t)

    @staticmethod
    def _grid(origin, cell_size, dims):
        o = np.ascontiguousarray(np.asarray(origin, dtype=np.float32).reshape(3))
        d = np.ascontiguousarray(np.asarray(dims, dtype=np.uint32).reshape(3))
        return o, np.float32(cell_size), d

    def _check(self, st: int, what: str):
        if st != 0:
            raise OracleError(f"{what}: oracle status {st}")

    # -- steps ---------------------------------------------------------
    def cells(self, origin, cell_size, dims) -> int:
        o, h, d = self._grid(origin, cell_size, dims)
        out = ctypes.c_uint64(0)
        st = self._lib.ugp_oracle_check_grid(self._p(o, _f32p), h, self._p(d, _u32p), ctypes.byref(out))
        self._check(st, "check_grid")
        return int(out.value)

    def check_grid(self, origin, cell_size, dims) -> int:
        o, h, d = self._grid(origin, cell_size, dims)
        out = ctypes.c_uint64(0)
        return int(self._lib.ugp_oracle_check_grid(self._p(o, _f32p), h, self._p(d, _u32p), ctypes.byref(out)))

    def cell_index(self, particles, origin, cell_size, dims, morton: bool = False) -> np.ndarray:
        p = np.ascontiguousarray(particles, dtype=np.float32).reshape(-1, 8)
        o, h, d = self._grid(origin, cell_size, dims)
        n = p.shape[0]
        out = np.empty(n, dtype=np.uint32)
        if morton:
            st = self._lib.ugp_oracle_cell_key(self._p(p, _f32p), n, self._p(o, _f32p), h, self._p(d, _u32p),
                                               ORDER_MORTON, self._p(out, _u32p))
        else:
            st = self._lib.ugp_oracle_cell_index(self._p(p, _f32p), n, self._p(o, _f32p), h, self._p(d, _u32p),
                                                 self._p(out, _u32p))
        self._check(st, "cell_index")
        return out

    def key_count(self, origin, cell_size, dims, morton: bool = False) -> int:
        o, h, d = self._grid(origin, cell_size, dims)
        out = ctypes.c_uint64(0)
        st = self._lib.ugp_oracle_key_count(self._p(o, _f32p), h, self._p(d, _u32p),
                                            ORDER_MORTON if morton else ORDER_LINEAR, ctypes.byref(out))
        self._check(st, "key_count")
        return int(out.value)

    def morton_bits(self, dims) -> int:
        d = np.ascontiguousarray(np.asarray(dims, dtype=np.uint32).reshape(3))
        b = ctypes.c_uint32(0)
        k = ctypes.c_uint64(0)
        self._check(self._lib.ugp_oracle_morton_bits(self._p(d, _u32p), ctypes.byref(b), ctypes.byref(k)),
                    "morton_bits")
        return int(b.value)

    def morton_keys(self, k3, bits: int) -> np.ndarray:
        k = np.ascontiguousarray(np.asarray(k3, dtype=np.uint32).reshape(-1, 3))
        out = np.empty(k.shape[0], dtype=np.uint32)
        self._check(self._lib.ugp_oracle_morton_keys(self._p(k, _u32p), k.shape[0], bits, self._p(out, _u32p)),
                    "morton_keys")
        return out

    def histogram(self, celdaDe, cells: int) -> np.ndarray:
        k = np.ascontiguousarray(celdaDe, dtype=np.uint32)
        out = np.empty(cells, dtype=np.uint32)
        st = self._lib.ugp_oracle_histogram(self._p(k, _u32p), k.size, cells, self._p(out, _u32p))
        self._check(st, "histogram")
        return out

    def exclusive_scan(self, conteos) -> np.ndarray:
        c = np.ascontiguousarray(conteos, dtype=np.uint32)
        out = np.empty(c.size + 1, dtype=np.uint32)
        st = self._lib.ugp_oracle_exclusive_scan(self._p(c, _u32p), c.size, self._p(out, _u32p))
        self._check(st, "exclusive_scan")
        return out

    def scatter(self, celdaDe, inicios) -> np.ndarray:
        k = np.ascontiguousarray(celdaDe, dtype=np.uint32)
        s = np.ascontiguousarray(inicios, dtype=np.uint32)
        cells = s.size - 1
        cur = np.empty(max(cells, 1), dtype=np.uint32)
        out = np.empty(k.size, dtype=np.uint32)
        st = self._lib.ugp_oracle_scatter(self._p(k, _u32p), k.size, self._p(s, _u32p), cells, self._p(cur, _u32p), self._p(out, _u32p))
        self._check(st, "scatter")
        return out

    def reorder(self, particles, ordenado) -> np.ndarray:
        p = np.ascontiguousarray(particles, dtype=np.float32).reshape(-1, 8)
        o = np.ascontiguousarray(ordenado, dtype=np.uint32)
        out = np.empty_like(p)
        st = self._lib.ugp_oracle_reorder(self._p(p, _f32p), self._p(o, _u32p), o.size, self._p(out, _f32p))
        self._check(st, "reorder")
        return out

    def grid_build(self, particles, origin, cell_size, dims, morton: bool = False) -> "GridIndex":
        p = np.ascontiguousarray(particles, dtype=np.float32).reshape(-1, 8)
        o, h, d = self._grid(origin, cell_size, dims)
        cells = self.key_count(o, h, d, morton)
        n = p.shape[0]
        celdaDe = np.empty(n, dtype=np.uint32)
        conteos = np.empty(cells, dtype=np.uint32)
        inicios = np.empty(cells + 1, dtype=np.uint32)
        ordenado = np.empty(n, dtype=np.uint32)
        reordered = np.empty_like(p)
        cursor = np.empty(max(cells, 1), dtype=np.uint32)
        st = self._lib.ugp_oracle_grid_build_keyed(
            self._p(p, _f32p), n, self._p(o, _f32p), h, self._p(d, _u32p),
            ORDER_MORTON if morton else ORDER_LINEAR, self._p(celdaDe, _u32p), self._p(conteos, _u32p), self._p(inicios, _u32p),
            self._p(ordenado, _u32p), self._p(reordered, _f32p), self._p(cursor, _u32p),
        )
        self._check(st, "grid_build")
        return GridIndex(celdaDe, conteos, inicios, ordenado, reordered)

    def alloc_build(self, n: int, cells: int) -> dict:
        """Output arrays (and the scatter's cursor) for timed_stages, allocated once."""
        return {"celdaDe": np.empty(n, dtype=np.uint32), "conteos": np.empty(cells, dtype=np.uint32),
                "inicios": np.empty(cells + 1, dtype=np.uint32), "ordenado": np.empty(n, dtype=np.uint32),
                "reordered": np.empty((n, 8), dtype=np.float32), "cursor": np.empty(max(cells, 1), dtype=np.uint32)}

    def timed_stages(self, particles, origin, cell_size, dims, bufs: dict) -> dict:
        """One linear-keyed build into preallocated `bufs` (alloc_build), each
        step timed on its own with a monotonic clock: count (cell keys, then
        the histogram), scan, scatter, reorder. Returns seconds per step."""
        import time

        p = np.ascontiguousarray(particles, dtype=np.float32).reshape(-1, 8)
        o, h, d = self._grid(origin, cell_size, dims)
        n = p.shape[0]
        cells = bufs["conteos"].size
        lib = self._lib
        pp, po, pd = self._p(p, _f32p), self._p(o, _f32p), self._p(d, _u32p)
        k, c, s = (self._p(bufs[x], _u32p) for x in ("celdaDe", "conteos", "inicios"))
        r, cur, out = self._p(bufs["ordenado"], _u32p), self._p(bufs["cursor"], _u32p), self._p(bufs["reordered"], _f32p)
        clock = time.perf_counter
        t0 = clock()
        st = lib.ugp_oracle_cell_index(pp, n, po, h, pd, k)
        st = st or lib.ugp_oracle_histogram(k, n, cells, c)
        t1 = clock()
        st = st or lib.ugp_oracle_exclusive_scan(c, cells, s)
        t2 = clock()
        st = st or lib.ugp_oracle_scatter(k, n, s, cells, cur, r)
        t3 = clock()
        st = st or lib.ugp_oracle_reorder(pp, r, n, out)
        t4 = clock()
        self._check(st, "timed_stages")
        return {"count": t1 - t0, "scan": t2 - t1, "scatter": t3 - t2, "reorder": t4 - t3}

    def neighbor_count(self, particles, origin, cell_size, dims, radius: float, morton: bool = False,
                       index: "GridIndex | None" = None) -> np.ndarray:
        """Per particle (original order): other particles in the 27 cells around
        its cell within `radius` (binary32 squared distance)."""
        p = np.ascontiguousarray(particles, dtype=np.float32).reshape(-1, 8)
        o, h, d = self._grid(origin, cell_size, dims)
        if index is None:
            index = self.grid_build(p, o, h, d, morton=morton)
        ini = np.ascontiguousarray(index.inicios, dtype=np.uint32)
        ordn = np.ascontiguousarray(index.ordenado, dtype=np.uint32)
        out = np.empty(p.shape[0], dtype=np.uint32)
        st = self._lib.ugp_oracle_neighbor_count(
            self._p(p, _f32p), p.shape[0], self._p(o, _f32p), h, self._p(d, _u32p),
            ORDER_MORTON if morton else ORDER_LINEAR, self._p(ini, _u32p), self._p(ordn, _u32p),
            np.float32(radius), self._p(out, _u32p))
        self._check(st, "neighbor_count")
        return out

    def gather(self, src: np.ndarray, idx) -> np.ndarray:
        """dst[k] = src[idx[k]] for arrays of fixed-size rows, byte for byte."""
        a = np.ascontiguousarray(src)
        i = np.ascontiguousarray(idx, dtype=np.uint32)
        rows = a.shape[0]
        eb = a.nbytes // rows if rows else a.itemsize * int(np.prod(a.shape[1:]))
        out = np.empty((i.size,) + a.shape[1:], dtype=a.dtype)
        st = self._lib.ugp_oracle_gather_bytes(a.ctypes.data, rows, eb, self._p(i, _u32p), i.size, out.ctypes.data)
        self._check(st, "gather")
        return out

    def diag(self, conteos, capacity: int) -> tuple[int, int]:
        c = np.ascontiguousarray(conteos, dtype=np.uint32)
        mx = ctypes.c_uint32(0)
        ov = ctypes.c_uint32(0)
        st = self._lib.ugp_oracle_diag(self._p(c, _u32p), c.size, capacity, ctypes.byref(mx), ctypes.byref(ov))
        self._check(st, "diag")
        return int(mx.value), int(ov.value)


@dataclass
class GridIndex:
    celdaDe: np.ndarray
    conteos: np.ndarray
    inicios: np.ndarray
    ordenado: np.ndarray
    reordered: np.ndarray


_default: Oracle | None = None


def load(rebuild: bool = False) -> Oracle:
    """The default oracle library, compiled on first use if absent or stale."""
    global _default
    if _default is not None and not rebuild:
        return _default
    stale = (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)
    if rebuild or stale:
        build()
    _default = Oracle(_LIB)
    return _default
