"""Seeded synthetic particle workloads for the uniform-grid index build.

This module only *draws inputs*. It holds none of the index build's
arithmetic (no cell keys, no counting, no prefix sums), so both the CPU
oracle and the GPU library can be fed from it without sharing any of the
method's code.

Record layout (page "El estado de las partículas en storage buffers",
section "La estructura y su alineación"): 32 bytes per particle, eight
float32 values ``[pos.x, pos.y, pos.z, vida, vel.x, vel.y, vel.z, masa]``.

Initial-state distribution (same page and section, the JavaScript
initialiser): each coordinate is ``(U - 0.5) * 10`` so positions cover
``[-5, 5)^3``; ``vida = 1 + 3U``; ``vel = 0``; ``masa = 0.5 + U``. The page
computes each value in double precision and stores it once into a
``Float32Array``; here every value is drawn in float64 and rounded to
float32 exactly once, the same way. ``U`` comes from NumPy's PCG64.

Draw order inside one workload: positions ``(N, 3)``, then ``vida (N,)``,
then ``masa (N,)``.

The grid of every named workload covers ``[-5, 5]^3`` with ``d^3`` cubic
cells: ``origin = (-5, -5, -5)``, ``cell_size = 10 / d``. For
d in {16, 128, 256} the cell size is an exact binary fraction in float32.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

RECORD_FLOATS = 8
RECORD_BYTES = 32

__all__ = [
    "Workload",
    "CONFIGS",
    "make_config",
    "make_uniform",
    "make_contention",
    "make_boundary_probe",
    "make_cell_centres",
    "make_worked_example",
    "make_sph_like",
    "SPH_RADIUS_FRACTION",
]


@dataclass
class Workload:
    """One synthetic input: particles plus the grid they are binned on."""

    name: str
    particles: np.ndarray  # (N, 8) float32, C-contiguous
    origin: np.ndarray  # (3,) float32
    cell_size: np.float32
    dims: np.ndarray  # (3,) uint32
    seed: int | None = None
    meta: dict = field(default_factory=dict)

    @property
    def n(self) -> int:
        return int(self.particles.shape[0])

    @property
    def cells(self) -> int:
        return int(np.prod(self.dims.astype(np.uint64)))


# name -> (seed, N, d); the construction is "uniform" unless stated.
CONFIGS = {
    "tiny": (1, 4096, 16),
    "sparse": (2, 100_000, 128),
    "baseline": (3, 1_000_000, 128),
    "contention": (4, 1_000_000, 128),
    "large": (5, 16_777_216, 256),
}


def _cube_grid(d: int):
    origin = np.full(3, -5.0, dtype=np.float32)
    cell_size = np.float32(10.0 / d)
    dims = np.full(3, d, dtype=np.uint32)
    return origin, cell_size, dims


def _records(pos64: np.ndarray, rng: np.random.Generator) -> np.ndarray:
    """Assemble (N, 8) float32 records from float64 positions; draws vida then masa."""
    n = pos64.shape[0]
    out = np.zeros((n, RECORD_FLOATS), dtype=np.float32)
    out[:, 0:3] = pos64.astype(np.float32)
    out[:, 3] = (1.0 + 3.0 * rng.random(n)).astype(np.float32)  # vida
    # vel stays 0 (columns 4..6)
    out[:, 7] = (0.5 + rng.random(n)).astype(np.float32)  # masa
    return out


def make_uniform(n: int, d: int, seed: int, name: str = "uniform") -> Workload:
    """Uniform positions in [-5, 5)^3 on a d^3 grid over [-5, 5]^3."""
    rng = np.random.Generator(np.random.PCG64(seed))
    pos = (rng.random((n, 3)) - 0.5) * 10.0
    parts = _records(pos, rng)
    origin, h, dims = _cube_grid(d)
    return Workload(name, parts, origin, h, dims, seed)


def make_contention(
    n: int = 1_000_000,
    d: int = 128,
    seed: int = 4,
    hot: int = 10_000,
    clusters: int = 4,
    per_cluster: int = 150_000,
    sigma: float = 0.3,
    outside: int = 50_000,
    name: str = "contention",
) -> Workload:
    """Skewed workload: one hot cell, Gaussian clusters, out-of-domain points.

    Draw order: hot-cell index and offsets, cluster centres and samples,
    out-of-domain points, uniform background, vida, masa, final shuffle.

    * ``hot`` particles sit strictly inside one random cell
      (offset 0.25..0.75 of a cell on every axis, far from any boundary
      compared with float32 rounding), so all of them share one counter.
    * ``clusters`` isotropic Gaussian clouds (std ``sigma``) with centres
      uniform in [-4, 4]^3; some samples leave the domain.
    * ``outside`` particles are uniform in [-5, 5)^3 except one random
      axis, which is pushed to a magnitude in (5.001, 6] with a random
      sign, so they lie strictly outside the domain after float32 rounding.
    * the rest are uniform in [-5, 5)^3.
    * the records are shuffled, so the hot cell's particles are spread
      over the whole array.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    origin, h, dims = _cube_grid(d)
    h64 = 10.0 / d
    o64 = -5.0
    k_hot = rng.integers(0, d, size=3)
    hot_pos = o64 + (k_hot[None, :] + 0.25 + 0.5 * rng.random((hot, 3))) * h64
    centres = rng.uniform(-4.0, 4.0, size=(clusters, 3))
    clus = centres[:, None, :] + sigma * rng.standard_normal((clusters, per_cluster, 3))
    clus = clus.reshape(-1, 3)
    out = (rng.random((outside, 3)) - 0.5) * 10.0
    axis = rng.integers(0, 3, size=outside)
    sign = np.where(rng.random(outside) < 0.5, -1.0, 1.0)
    mag = 5.001 + (1.0 - rng.random(outside)) * 0.999
    out[np.arange(outside), axis] = sign * mag
    rest = n - hot - clusters * per_cluster - outside
    if rest < 0:
        raise ValueError("contention workload: parts exceed n")
    back = (rng.random((rest, 3)) - 0.5) * 10.0
    pos = np.concatenate([hot_pos, clus, out, back], axis=0)
    parts = _records(pos, rng)
    perm = rng.permutation(n)
    parts = np.ascontiguousarray(parts[perm])
    meta = {"hot_cell_xyz": [int(v) for v in k_hot], "hot": hot, "outside": outside}
    return Workload(name, parts, origin, h, dims, seed, meta)


def make_config(name: str, seed: int | None = None) -> Workload:
    """Named workload: tiny, sparse, baseline, contention or large."""
    key = name.lower()
    if key not in CONFIGS:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}")
    s0, n, d = CONFIGS[key]
    s = s0 if seed is None else seed
    if key == "contention":
        return make_contention(n=n, d=d, seed=s, name=key)
    return make_uniform(n, d, s, name=key)


# Neighbour-query workload: 1,000,000 uniform particles on 32^3 cells gives
# 30.5 particles per cell (inside the 20-60 per cell of a well-resolved fluid
# on the counting page, section on dense-cell contention), and a radius of
# 0.87 cell gives (4/3) pi 0.87^3 * 30.5 ~ 84 neighbours per particle, the
# SPH figure on the reorder page (section "Qué cuesta la indirección").
SPH_RADIUS_FRACTION = 0.87


def make_sph_like(n: int = 1_000_000, d: int = 32, seed: int = 6) -> Workload:
    """Uniform particles at SPH-like density for the 27-cell neighbour query."""
    return make_uniform(n, d, seed, name="sph_like")


def make_boundary_probe(
    dims, origin, cell_size, seed: int = 11, per_axis_random: int = 2048
) -> Workload:
    """Positions on, and one float32 step either side of, every cell face.

    For each axis a and each face index k in 0..dims[a], the coordinate on
    that axis is ``fl32(origin[a] + k * cell_size)`` and its two float32
    neighbours; the other two coordinates are drawn uniformly inside the
    domain. Random float32 values within 4 ulp of faces are added, plus
    the face values just outside the domain on both sides. These are the
    inputs where an approximate division or a wrong rounding order picks
    a different cell.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    dims = np.asarray(dims, dtype=np.uint32)
    origin = np.asarray(origin, dtype=np.float32)
    h = np.float32(cell_size)
    rows = []
    lo = origin.astype(np.float64)
    hi = lo + dims.astype(np.float64) * float(h)
    for a in range(3):
        k = np.arange(int(dims[a]) + 1, dtype=np.float64)
        face = (lo[a] + k * float(h)).astype(np.float32)
        vals = np.concatenate(
            [
                face,
                np.nextafter(face, np.float32(-np.inf)),
                np.nextafter(face, np.float32(np.inf)),
            ]
        )
        # random values within 4 ulp of a random face
        pick = face[rng.integers(0, face.size, per_axis_random)]
        steps = rng.integers(-4, 5, per_axis_random)
        jit = pick.copy()
        for s in range(1, 5):
            up = steps >= s
            dn = steps <= -s
            jit[up] = np.nextafter(jit[up], np.float32(np.inf))
            jit[dn] = np.nextafter(jit[dn], np.float32(-np.inf))
        vals = np.concatenate([vals, jit]).astype(np.float32)
        m = vals.size
        pos = np.empty((m, 3), dtype=np.float32)
        for b in range(3):
            pos[:, b] = (lo[b] + rng.random(m) * (hi[b] - lo[b])).astype(np.float32)
        pos[:, a] = vals
        rows.append(pos)
    pos = np.concatenate(rows, axis=0)
    n = pos.shape[0]
    parts = np.zeros((n, RECORD_FLOATS), dtype=np.float32)
    parts[:, 0:3] = pos
    parts[:, 3] = (1.0 + 3.0 * rng.random(n)).astype(np.float32)
    parts[:, 7] = (0.5 + rng.random(n)).astype(np.float32)
    perm = rng.permutation(n)
    parts = np.ascontiguousarray(parts[perm])
    return Workload("boundary_probe", parts, origin, h, dims, seed)


def make_cell_centres(dims, origin, cell_size, cells_xyz) -> Workload:
    """One particle at the centre of each listed cell (kx, ky, kz)."""
    dims = np.asarray(dims, dtype=np.uint32)
    origin = np.asarray(origin, dtype=np.float32)
    h = np.float32(cell_size)
    k = np.asarray(cells_xyz, dtype=np.float64).reshape(-1, 3)
    pos = origin.astype(np.float64)[None, :] + (k + 0.5) * float(h)
    parts = np.zeros((k.shape[0], RECORD_FLOATS), dtype=np.float32)
    parts[:, 0:3] = pos.astype(np.float32)
    parts[:, 3] = 1.0
    parts[:, 7] = 1.0
    return Workload("cell_centres", parts, origin, h, dims, None)


def make_worked_example(conteos, seed: int = 7) -> Workload:
    """A shuffled particle set on a 1-D row of cells realising given counts.

    ``dims = (len(conteos), 1, 1)``, ``origin = 0``, ``cell_size = 1``;
    cell c receives ``conteos[c]`` particles at ``(c + 0.5, 0.5, 0.5)``.
    Each record's ``vida`` holds its cell number and ``masa`` its
    position in the pre-shuffle order, so records are distinguishable.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    conteos = [int(v) for v in conteos]
    rows = []
    serial = 0
    for c, cnt in enumerate(conteos):
        for _ in range(cnt):
            rows.append([c + 0.5, 0.5, 0.5, float(c), 0.0, 0.0, 0.0, float(serial)])
            serial += 1
    parts = np.asarray(rows, dtype=np.float32).reshape(-1, RECORD_FLOATS)
    perm = rng.permutation(parts.shape[0])
    parts = np.ascontiguousarray(parts[perm])
    origin = np.zeros(3, dtype=np.float32)
    dims = np.asarray([len(conteos), 1, 1], dtype=np.uint32)
    return Workload("worked_example", parts, origin, np.float32(1.0), dims, seed)
