"""Uniform-grid particle index build on MI355X: Python binding of libugp.so.

Argument marshalling only. Every step of the build runs in the HIP
kernels of ``csrc/ugp.hip`` behind the C ABI of ``include/ugp.h``; PyTorch
supplies device memory and the current stream. There is no CPU fallback:
if the library is not built, or the tensors are not on a GPU, the calls
raise.

The names follow the C ABI (``grid_build`` is ``ugp_grid_build``, etc.).
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libugp.so")

UGP_OK = 0
UGP_ERR_NULL = -1
UGP_ERR_ARG = -2
UGP_ERR_RANGE = -3
UGP_ERR_ALIAS = -4
UGP_ERR_ALIGN = -5
UGP_ERR_WORKSPACE = -6
UGP_ERR_HIP = -7

FLAG_STABLE = 0x1
FLAG_GATHER = 0x2
FLAG_MORTON = 0x4
FLAG_INDEX_ONLY = 0x8

NUM_STAGES = 6  # stage slots; names depend on the path, see stage_names()

_vp = ctypes.c_void_p
_u32 = ctypes.c_uint32
_u32_3 = _u32 * 3
_f32_3 = ctypes.c_float * 3

_lib = None


class ArrayDesc(ctypes.Structure):
    """ugp_array_desc: one array of a split state."""

    _fields_ = [("src", ctypes.c_void_p), ("dst", ctypes.c_void_p), ("elem_bytes", ctypes.c_uint32)]


class UGPError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def library_path() -> str:
    return LIB_PATH


def load_library():
    """Load libugp.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"HIP library not built: {LIB_PATH} is missing "
            "(run `python -c 'import __graft_entry__ as g; g.build()'` first)"
        )
    lib = ctypes.CDLL(LIB_PATH)
    lib.ugp_abi_version.restype = ctypes.c_int
    lib.ugp_abi_version.argtypes = []
    lib.ugp_status_string.restype = ctypes.c_char_p
    lib.ugp_status_string.argtypes = [ctypes.c_int]
    lib.ugp_grid_key_count.restype = ctypes.c_int
    lib.ugp_grid_key_count.argtypes = [ctypes.POINTER(_u32), _u32, ctypes.POINTER(ctypes.c_uint64)]
    lib.ugp_grid_workspace_bytes.restype = ctypes.c_int
    lib.ugp_grid_workspace_bytes.argtypes = [_u32, ctypes.POINTER(_u32), _u32, ctypes.POINTER(ctypes.c_size_t)]
    build_args = [_vp, _u32, ctypes.POINTER(ctypes.c_float), ctypes.c_float, ctypes.POINTER(_u32),
                  _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _u32, _vp]
    lib.ugp_grid_build.restype = ctypes.c_int
    lib.ugp_grid_build.argtypes = build_args
    lib.ugp_grid_build_stage.restype = ctypes.c_int
    lib.ugp_grid_build_stage.argtypes = [_u32, *build_args]
    lib.ugp_grid_build_timed.restype = ctypes.c_int
    lib.ugp_grid_build_timed.argtypes = [*build_args, _u32, _vp, _vp]
    lib.ugp_grid_build_diag.restype = ctypes.c_int
    lib.ugp_grid_build_diag.argtypes = [*build_args[:-2], _u32, _vp, _u32, _vp]
    lib.ugp_grid_build_noalloc.restype = ctypes.c_int
    lib.ugp_grid_build_noalloc.argtypes = [*build_args[:10], _u32, _vp]
    lib.ugp_neighbor_count.restype = ctypes.c_int
    lib.ugp_neighbor_count.argtypes = [_vp, _u32, ctypes.POINTER(ctypes.c_float), ctypes.c_float,
                                       ctypes.POINTER(_u32), _vp, _vp, ctypes.c_float, _vp, _u32, _vp]
    lib.ugp_reorder_arrays.restype = ctypes.c_int
    lib.ugp_reorder_arrays.argtypes = [_vp, _u32, _u32, ctypes.POINTER(ArrayDesc), _u32, _vp]
    lib.ugp_cell_diag.restype = ctypes.c_int
    lib.ugp_cell_diag.argtypes = [_vp, _u32, _u32, _vp, _vp]
    lib.ugp_cell_diag_timed.restype = ctypes.c_int
    lib.ugp_cell_diag_timed.argtypes = [_vp, _u32, _u32, _vp, _vp, _vp, _vp]
    lib.ugp_grid_stage_name.restype = ctypes.c_char_p
    lib.ugp_grid_stage_name.argtypes = [_u32, ctypes.POINTER(_u32), _u32, _u32]
    lib.ugp_scan_workspace_bytes.restype = ctypes.c_int
    lib.ugp_scan_workspace_bytes.argtypes = [_u32, ctypes.POINTER(ctypes.c_size_t)]
    lib.ugp_exclusive_scan_u32.restype = ctypes.c_int
    lib.ugp_exclusive_scan_u32.argtypes = [_vp, _u32, _vp, _vp, ctypes.c_size_t, _vp]
    lib.ugp_reorder.restype = ctypes.c_int
    lib.ugp_reorder.argtypes = [_vp, _u32, _vp, _u32, _vp, _vp]
    if lib.ugp_abi_version() != 1:
        raise RuntimeError("libugp.so ABI version mismatch")
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().ugp_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != UGP_OK:
        raise UGPError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(device: torch.device, stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _require_gpu(t: torch.Tensor, name: str, dtype: Optional[torch.dtype], device: Optional[torch.device] = None):
    """A contiguous GPU tensor of `dtype` (None: any), on `device` if given."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other arrays on {device}")


def _on(device: torch.device):
    """The library launches on the current device: make it the arrays' one."""
    return torch.cuda.device(device)


def _alloc_on(device: torch.device, stream):
    """Context for allocating what a call on `stream` reads or writes: the
    caching allocator then ties those blocks to that stream, so memory freed
    when the call returns is not handed to work on another stream while the
    call may still be running. No stream: the current one, as the call uses."""
    import contextlib

    if stream is None:
        return contextlib.nullcontext()
    return torch.cuda.stream(stream)


def _dims3(dims) -> tuple[int, int, int]:
    d = tuple(int(v) for v in dims)
    if len(d) != 3:
        raise ValueError("dims must have 3 entries")
    return d


def key_count(dims: Sequence[int], flags: int = 0) -> int:
    """Entries of conteos (inicios has one more) for this grid and flags."""
    lib = load_library()
    d = _u32_3(*_dims3(dims))
    out = ctypes.c_uint64(0)
    _check(lib.ugp_grid_key_count(d, int(flags), ctypes.byref(out)), "ugp_grid_key_count")
    return int(out.value)


def _flags(stable: bool, gather: bool, morton: bool) -> int:
    return (FLAG_STABLE if stable else 0) | (FLAG_GATHER if gather else 0) | (FLAG_MORTON if morton else 0)


def workspace_bytes(n: int, dims: Sequence[int], flags: int = 0) -> int:
    lib = load_library()
    d = _u32_3(*_dims3(dims))
    out = ctypes.c_size_t(0)
    _check(lib.ugp_grid_workspace_bytes(int(n), d, int(flags), ctypes.byref(out)), "ugp_grid_workspace_bytes")
    return int(out.value)


def stage_names(n: int, dims: Sequence[int], flags: int = 0) -> list:
    """Names of the stage slots for this shape and flags (None = slot unused)."""
    lib = load_library()
    d = _u32_3(*_dims3(dims))
    out = []
    for st in range(NUM_STAGES):
        name = lib.ugp_grid_stage_name(int(n), d, int(flags), st)
        out.append(None if name is None else name.decode())
    return out


@dataclass
class GridIndex:
    """Outputs of one build (all GPU tensors)."""

    celdaDe: torch.Tensor  # (N,) int32 storage of u32 cell indices
    conteos: torch.Tensor  # (C,) u32 histogram
    inicios: torch.Tensor  # (C+1,) u32 starts, inicios[C] = N
    ordenado: torch.Tensor  # (N,) u32 particle indices grouped by cell
    reordered: torch.Tensor  # (N, 8) float32 records in cell order


def alloc_outputs(n: int, dims: Sequence[int], device, flags: int = 0, stream=None):
    """Output tensors and the workspace for one build (torch allocations),
    tied to `stream` (default: the current stream)."""
    return _fill_in(n, dims, device, flags, None, None, stream)


def _fill_in(n: int, dims, device, flags: int, out: Optional[GridIndex], workspace: Optional[torch.Tensor],
             stream=None):
    """Allocate the outputs and/or the workspace the caller did not pass, on
    the stream the build is enqueued on."""
    d = _dims3(dims)
    dev = torch.device(device)
    with _alloc_on(dev, stream):
        return _fill_in_now(n, d, dev, flags, out, workspace)


def _fill_in_now(n: int, d, dev, flags: int, out: Optional[GridIndex], workspace: Optional[torch.Tensor]):
    if out is None:
        cells = key_count(d, flags)
        out = GridIndex(
            celdaDe=torch.empty(n, dtype=torch.int32, device=dev),
            conteos=torch.empty(cells, dtype=torch.int32, device=dev),
            inicios=torch.empty(cells + 1, dtype=torch.int32, device=dev),
            ordenado=torch.empty(n, dtype=torch.int32, device=dev),
            reordered=torch.empty((0 if flags & FLAG_INDEX_ONLY else n, 8), dtype=torch.float32, device=dev),
        )
    if workspace is None:
        workspace = torch.empty(max(workspace_bytes(n, d, flags), 256), dtype=torch.uint8, device=dev)
    return out, workspace


def _build_args(particles, origin, cell_size, dims, out: GridIndex, workspace, flags, stream):
    _require_gpu(particles, "particles", torch.float32)
    if particles.dim() != 2 or particles.shape[1] != 8:
        raise ValueError("particles must have shape (N, 8) (32-byte records)")
    dev = particles.device
    n = int(particles.shape[0])
    d = _dims3(dims)
    for name in ("celdaDe", "conteos", "inicios", "ordenado"):
        _require_gpu(getattr(out, name), name, torch.int32, dev)
    index_only = bool(flags & FLAG_INDEX_ONLY)
    if not index_only:
        _require_gpu(out.reordered, "reordered", torch.float32, dev)
    if workspace is not None:  # None: the no-allocation entry point, which takes none
        _require_gpu(workspace, "workspace", torch.uint8, dev)
    cells = key_count(d, flags)
    if out.celdaDe.numel() < n or out.ordenado.numel() < n or (not index_only and out.reordered.numel() < 8 * n):
        raise ValueError("per-particle outputs are smaller than N")
    if out.conteos.numel() < cells or out.inicios.numel() < cells + 1:
        raise ValueError("per-cell outputs are smaller than the cell count")
    o = _f32_3(*[float(v) for v in origin])
    return [
        _ptr(particles), n, o, ctypes.c_float(float(cell_size)), _u32_3(*d),
        _ptr(out.celdaDe), _ptr(out.conteos), _ptr(out.inicios), _ptr(out.ordenado),
        None if index_only else _ptr(out.reordered), _ptr(workspace),
        ctypes.c_size_t(0 if workspace is None else workspace.numel()),
        int(flags), _stream_handle(particles.device, stream),
    ]


def grid_build(
    particles: torch.Tensor,
    origin: Sequence[float],
    cell_size: float,
    dims: Sequence[int],
    *,
    stable: bool = False,
    gather: bool = False,
    morton: bool = False,
    index_only: bool = False,
    out: Optional[GridIndex] = None,
    workspace: Optional[torch.Tensor] = None,
    stream=None,
) -> GridIndex:
    """ugp_grid_build on torch tensors; enqueued on the current stream.
    index_only: build the index without writing `reordered`."""
    lib = load_library()
    flags = _flags(stable, gather, morton) | (FLAG_INDEX_ONLY if index_only else 0)
    n = int(particles.shape[0])
    out, workspace = _fill_in(n, dims, particles.device, flags, out, workspace, stream)
    args = _build_args(particles, origin, cell_size, dims, out, workspace, flags, stream)
    with _on(particles.device):
        _check(lib.ugp_grid_build(*args), "ugp_grid_build")
    return out


NOALLOC_SCRATCH_BYTES = 48 << 20  # UGP_NOALLOC_SCRATCH_BYTES


def grid_build_noalloc(
    particles: torch.Tensor,
    origin: Sequence[float],
    cell_size: float,
    dims: Sequence[int],
    out: GridIndex,
    *,
    stable: bool = False,
    gather: bool = False,
    morton: bool = False,
    index_only: bool = False,
    stream=None,
) -> GridIndex:
    """ugp_grid_build_noalloc: the build into caller-given outputs with the
    library's own fixed device workspace (nothing is allocated). Calls that
    overlap on one GPU race on that workspace."""
    lib = load_library()
    flags = _flags(stable, gather, morton) | (FLAG_INDEX_ONLY if index_only else 0)
    args = _build_args(particles, origin, cell_size, dims, out, None, flags, stream)
    with _on(particles.device):
        _check(lib.ugp_grid_build_noalloc(*args[:10], args[12], args[13]), "ugp_grid_build_noalloc")
    return out


def grid_build_diag(
    particles: torch.Tensor,
    origin: Sequence[float],
    cell_size: float,
    dims: Sequence[int],
    capacity: int,
    *,
    diag: Optional[torch.Tensor] = None,
    stable: bool = False,
    gather: bool = False,
    morton: bool = False,
    out: Optional[GridIndex] = None,
    workspace: Optional[torch.Tensor] = None,
    stream=None,
) -> tuple[GridIndex, torch.Tensor]:
    """ugp_grid_build_diag: the build plus the overflow diagnostics in `diag`
    (2 u32 on the GPU: largest cell occupancy, insertions past `capacity`)."""
    lib = load_library()
    flags = _flags(stable, gather, morton)
    n = int(particles.shape[0])
    out, workspace = _fill_in(n, dims, particles.device, flags, out, workspace, stream)
    if diag is None:
        with _alloc_on(particles.device, stream):
            diag = torch.empty(2, dtype=torch.int32, device=particles.device)
    _require_gpu(diag, "diag", torch.int32, particles.device)
    if diag.numel() < 2:
        raise ValueError("diag needs 2 entries")
    args = _build_args(particles, origin, cell_size, dims, out, workspace, flags, stream)
    with _on(particles.device):
        _check(lib.ugp_grid_build_diag(*args[:-2], int(capacity), _ptr(diag), *args[-2:]), "ugp_grid_build_diag")
    return out, diag


def cell_diag(conteos: torch.Tensor, capacity: int, out: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """ugp_cell_diag: overflow diagnostics of an existing histogram."""
    lib = load_library()
    _require_gpu(conteos, "conteos", torch.int32)
    if out is None:
        with _alloc_on(conteos.device, stream):
            out = torch.empty(2, dtype=torch.int32, device=conteos.device)
    _require_gpu(out, "out", torch.int32, conteos.device)
    if out.numel() < 2:
        raise ValueError("out needs 2 entries")
    with _on(conteos.device):
        st = lib.ugp_cell_diag(_ptr(conteos), int(conteos.numel()), int(capacity), _ptr(out),
                               _stream_handle(conteos.device, stream))
    _check(st, "ugp_cell_diag")
    return out


def cell_diag_timed(conteos: torch.Tensor, capacity: int, event_before, event_after,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """ugp_cell_diag_timed: cell_diag with two torch.cuda.Event objects
    recorded at its kernel's own start and end."""
    lib = load_library()
    _require_gpu(conteos, "conteos", torch.int32)
    for ev in (event_before, event_after):
        if not getattr(ev, "cuda_event", 0):
            ev.record()  # torch creates the underlying event lazily
    if out is None:
        with _alloc_on(conteos.device, stream):
            out = torch.empty(2, dtype=torch.int32, device=conteos.device)
    _require_gpu(out, "out", torch.int32, conteos.device)
    if out.numel() < 2:
        raise ValueError("out needs 2 entries")
    with _on(conteos.device):
        st = lib.ugp_cell_diag_timed(_ptr(conteos), int(conteos.numel()), int(capacity), _ptr(out),
                                     _stream_handle(conteos.device, stream),
                                     ctypes.c_void_p(event_before.cuda_event),
                                     ctypes.c_void_p(event_after.cuda_event))
    _check(st, "ugp_cell_diag_timed")
    return out


def neighbor_count(particles: torch.Tensor, origin: Sequence[float], cell_size: float, dims: Sequence[int],
                   inicios: torch.Tensor, ordenado: Optional[torch.Tensor], radius: float, *,
                   morton: bool = False, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """ugp_neighbor_count: per-particle neighbour counts over the 27 cells.
    Pass the build's input with its ordenado, or its `reordered` output with
    ordenado=None (counts then follow the cell order)."""
    lib = load_library()
    _require_gpu(particles, "particles", torch.float32)
    if particles.dim() != 2 or particles.shape[1] != 8:
        raise ValueError("particles must have shape (N, 8)")
    n = int(particles.shape[0])
    d = _dims3(dims)
    flags = FLAG_MORTON if morton else 0
    dev = particles.device
    _require_gpu(inicios, "inicios", torch.int32, dev)
    if inicios.numel() < key_count(d, flags) + 1:
        raise ValueError("inicios is smaller than the key count + 1")
    if ordenado is not None:
        _require_gpu(ordenado, "ordenado", torch.int32, dev)
        if ordenado.numel() < n:
            raise ValueError("ordenado is smaller than N")
    if out is None:
        with _alloc_on(dev, stream):
            out = torch.empty(n, dtype=torch.int32, device=particles.device)
    _require_gpu(out, "out", torch.int32, dev)
    if out.numel() < n:
        raise ValueError("out is smaller than N")
    o = _f32_3(*[float(v) for v in origin])
    with _on(dev):
        st = lib.ugp_neighbor_count(_ptr(particles), n, o, ctypes.c_float(float(cell_size)), _u32_3(*d),
                                    _ptr(inicios), _ptr(ordenado), ctypes.c_float(float(radius)), _ptr(out), flags,
                                    _stream_handle(dev, stream))
    _check(st, "ugp_neighbor_count")
    return out


def grid_build_stage(stage: int, particles, origin, cell_size, dims, out: GridIndex, workspace,
                     *, flags: int = 0, stream=None) -> None:
    """ugp_grid_build_stage: enqueue one stage with the same arguments."""
    lib = load_library()
    args = _build_args(particles, origin, cell_size, dims, out, workspace, flags, stream)
    with _on(particles.device):
        _check(lib.ugp_grid_build_stage(int(stage), *args), f"ugp_grid_build_stage({stage})")


def grid_build_timed(stage: int, event_before, event_after, particles, origin, cell_size, dims,
                     out: GridIndex, workspace, *, flags: int = 0, stream=None) -> None:
    """ugp_grid_build_timed: full build, two torch.cuda.Event objects recorded
    around stage slot `stage` inside the same C call."""
    lib = load_library()
    for ev in (event_before, event_after):
        if not getattr(ev, "cuda_event", 0):
            ev.record()  # torch creates the underlying event lazily
    args = _build_args(particles, origin, cell_size, dims, out, workspace, flags, stream)
    with _on(particles.device):
        st = lib.ugp_grid_build_timed(*args, int(stage), ctypes.c_void_p(event_before.cuda_event),
                                      ctypes.c_void_p(event_after.cuda_event))
    _check(st, "ugp_grid_build_timed")


def exclusive_scan_u32(x: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """ugp_exclusive_scan_u32: out[0..n] with out[n] = total (mod 2^32)."""
    lib = load_library()
    _require_gpu(x, "x", torch.int32)
    n = int(x.numel())
    if out is None:
        with _alloc_on(x.device, stream):
            out = torch.empty(n + 1, dtype=torch.int32, device=x.device)
    _require_gpu(out, "out", torch.int32, x.device)
    if out.numel() < n + 1:
        raise ValueError("out needs n+1 entries")
    need = ctypes.c_size_t(0)
    _check(lib.ugp_scan_workspace_bytes(n, ctypes.byref(need)), "ugp_scan_workspace_bytes")
    with _alloc_on(x.device, stream):  # freed on return, while the scan may still run on `stream`
        ws = torch.empty(max(int(need.value), 256), dtype=torch.uint8, device=x.device)
    with _on(x.device):
        st = lib.ugp_exclusive_scan_u32(_ptr(x), n, _ptr(out), _ptr(ws), ctypes.c_size_t(ws.numel()),
                                        _stream_handle(x.device, stream))
    _check(st, "ugp_exclusive_scan_u32")
    return out


def reorder(src: torch.Tensor, idx: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """ugp_reorder: out[k] = src[idx[k]] (32-byte records, bit for bit)."""
    lib = load_library()
    _require_gpu(src, "src", torch.float32)
    _require_gpu(idx, "idx", torch.int32, src.device)
    if src.dim() != 2 or src.shape[1] != 8:
        raise ValueError("src must have shape (N, 8)")
    n = int(idx.numel())
    if out is None:
        with _alloc_on(src.device, stream):
            out = torch.empty((n, 8), dtype=torch.float32, device=src.device)
    _require_gpu(out, "out", torch.float32, src.device)
    if out.numel() < 8 * n:
        raise ValueError("out must hold one 32-byte record per index")
    with _on(src.device):
        st = lib.ugp_reorder(_ptr(src), int(src.shape[0]), _ptr(idx), n, _ptr(out),
                             _stream_handle(src.device, stream))
    _check(st, "ugp_reorder")
    return out


def reorder_arrays(idx: torch.Tensor, srcs: Sequence[torch.Tensor], outs: Optional[Sequence[torch.Tensor]] = None,
                   stream=None) -> list:
    """ugp_reorder_arrays: out_q[k] = src_q[idx[k]] for every array in one
    kernel. Each src is a contiguous GPU tensor whose first dimension indexes
    particles (an element is one row, any dtype, a multiple of 4 bytes)."""
    lib = load_library()
    _require_gpu(idx, "idx", torch.int32)
    n = int(idx.numel())
    if not srcs:
        raise ValueError("at least one array")
    n_src = int(srcs[0].shape[0])
    if outs is None:
        with _alloc_on(idx.device, stream):
            outs = [torch.empty((n,) + tuple(s.shape[1:]), dtype=s.dtype, device=s.device) for s in srcs]
    if len(outs) != len(srcs):
        raise ValueError("one output per array")
    descs = (ArrayDesc * len(srcs))()
    for q, (s, o) in enumerate(zip(srcs, outs)):
        for t, name in ((s, "src"), (o, "out")):
            _require_gpu(t, f"{name} {q}", None, idx.device)
        if int(s.shape[0]) != n_src:
            raise ValueError("every source needs the same number of rows")
        eb = s.element_size() * (s.numel() // max(1, s.shape[0]))
        if o.dtype != s.dtype or tuple(o.shape[1:]) != tuple(s.shape[1:]) or int(o.shape[0]) < n:
            raise ValueError(f"out {q} must match src {q} row shape and hold N rows")
        descs[q] = ArrayDesc(s.data_ptr(), o.data_ptr(), eb)
    with _on(idx.device):
        st = lib.ugp_reorder_arrays(_ptr(idx), n, n_src, descs, len(srcs), _stream_handle(idx.device, stream))
    _check(st, "ugp_reorder_arrays")
    return list(outs)


def as_u32_numpy(t: torch.Tensor):
    """Copy a u32-in-int32 GPU tensor to a NumPy uint32 array."""
    return t.detach().cpu().numpy().view("uint32")


__all__ = [
    "GridIndex", "UGPError", "alloc_outputs", "as_u32_numpy", "cell_diag", "exclusive_scan_u32", "grid_build",
    "grid_build_diag", "grid_build_noalloc", "neighbor_count", "reorder_arrays", "ArrayDesc", "FLAG_INDEX_ONLY",
    "grid_build_stage", "grid_build_timed", "library_path", "load_library", "reorder", "stage_names",
    "status_string", "workspace_bytes", "key_count", "FLAG_STABLE", "FLAG_GATHER", "FLAG_MORTON", "NUM_STAGES",
]
