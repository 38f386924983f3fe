"""Benchmark of the uniform-grid index build on one MI355X.

One step = one full build (cell keys and histogram, prefix sums, scatter
of particle indices, record reorder) over the Baseline workload: 1,000,000 uniform particles on 128^3 cells,
32-byte records, resident in HBM before timing starts.

Headline timing is cold: before every step a 1 GiB read-only pass evicts
the L2s and the 256 MiB Infinity Cache with clean lines (a write-based
flush would leave dirty lines whose write-back the next step would pay);
the flush sits outside the HIP events that bracket each step, and ms_per_step is the median of the K per-step
event times (mean, p10/p90 and the worst step are reported beside it). A warm figure (K back-to-back builds between one event pair) is
reported separately; at this size the whole working set fits in the
Infinity Cache, so warm numbers can exceed what HBM alone allows.

Per-stage durations come from HIP events that the library records at the
stage kernel's own start and end (hipExtLaunchKernel) inside a full cold
build (one C call, so no host work separates stages), K builds per slot,
median; the stage with the longest median is the dominant kernel, whose
kernel-I/O bytes / median duration is the roofline figure.

Prints ONE JSON line on stdout.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth, GB/s
METRIC = "grid-build particles/s (count+scan+scatter+reorder) and % of HBM peak, 1M@128^3"
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic_baseline_1M_128.txt")
KERNEL_DIR = os.path.join(ROOT, "uniform_grid_particle_amd", "csrc")

WORKLOAD_NAMES = {
    "tiny": "Tiny: 4,096 uniform particles on 16^3 cells",
    "sparse": "Sparse: 100,000 uniform particles on 128^3 cells",
    "baseline": "Baseline: 1,000,000 uniform particles on 128^3 cells",
    "contention": "Contention/clamp: 1,000,000 particles on 128^3 cells, one 10,000-particle cell, 4 clusters, 5% outside",
    "large": "Large SPH-like: 16,777,216 uniform particles on 256^3 cells",
}


def alg_bytes(n: int, c: int, mode: str) -> dict:
    """Bytes each kernel must move by design, each logical array counted once
    per kernel that touches it (32 B per record, 4 B per u32). The small
    row-block x tile matrices of the bucketed path are left out, and so is
    the stable fix-up, whose work depends on the input.

    The end-to-end figure uses the fixed model of the four page steps
    instead: 116 N + 16 C + 4 (see hbm_frac_e2e)."""
    move = mode in ("atomic", "stable")  # stable: the tile kernel still moves every record
    return {
        # staged path (cells <= 2^22, n <= 2^21)
        "chunk_sort": 72 * n,  # record read, celdaDe, chunk records + indices written
        "tile_sort": (36 * n + 4 * c + 4 * (c + 1) + 4 * n + (32 * n if move else 0)),
        # bucketed path (more particles or keys; tile_sort as above)
        "coarse_sort": 72 * n,  # as chunk_sort, by bucket
        "tile_scan": 4 * n,  # the packed index words read (count per tile)
        "rebucket": 72 * n,  # chunk records + indices read, written in tile order
        # direct path (larger grids)
        "clear": 4 * c,
        "count": 36 * n,
        "scan": 12 * c + 4,
        "scatter": 80 * n if move else 12 * n,
        # optional passes
        # data-dependent: on the tile paths only the cells the tile kernel
        # listed are touched (none on uniform inputs)
        "stable_sort": None,
        "gather": 68 * n,
    }


def _code_only(text: str) -> str:
    """A source file without its comments and blank lines (the sources hold no
    string literal with a comment marker in it)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", line).rstrip() for line in text.splitlines())
    return "\n".join(line for line in lines if line.strip())


def source_digest() -> str:
    """Digest of the code of every kernel source file, comments left out
    (traffic figures go stale with the code, not with its comments)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_DIR)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(KERNEL_DIR, name), encoding="utf-8") as f:
                h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel: str):
    """Measured HBM bytes per dispatch of `kernel`, from the committed counter
    summary, or None when absent or taken on a different kernel source."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    vals = {}
    with open(PROFILE_TRAFFIC, encoding="utf-8") as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != source_digest():
        return None
    key = f"{kernel}_bytes_per_dispatch"
    return float(vals[key]) if key in vals else None


def cpu_baseline(wl, budget_s: float):
    """The oracle as it stands, single-threaded and pinned to one core, on the
    same workload: each step (count = cell keys + histogram, scan, scatter,
    reorder) timed on its own into output arrays allocated once, repeated
    until the budget is spent (at least 3 builds); medians per step."""
    import oracle

    orc = oracle.load()
    bufs = orc.alloc_build(wl.n, wl.cells)
    pinned = None
    old_aff = None
    if hasattr(os, "sched_setaffinity"):
        old_aff = os.sched_getaffinity(0)
        pinned = min(old_aff)
        os.sched_setaffinity(0, {pinned})
    try:
        runs = []
        t_end = time.perf_counter() + budget_s
        while True:
            runs.append(orc.timed_stages(wl.particles, wl.origin, wl.cell_size, wl.dims, bufs))
            if time.perf_counter() >= t_end and len(runs) >= 3:
                break
    finally:
        if old_aff is not None:
            os.sched_setaffinity(0, old_aff)
    stage_s = {k: statistics.median(r[k] for r in runs) for k in runs[0]}
    total = statistics.median(sum(r.values()) for r in runs)
    return {
        "value": wl.n / total,
        "unit": "particles/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"full {wl.name} build ({wl.n} particles, {wl.cells} cells) repeated {len(runs)}x into "
                  f"preallocated outputs, median {total * 1e3:.1f} ms; single-threaded C oracle pinned to core "
                  f"{pinned}",
        "stages_ms": {k: round(v * 1e3, 3) for k, v in stage_s.items()},
        "stages_particles_per_s": {k: wl.n / v for k, v in stage_s.items() if v > 0},
        "host_cpu": _cpu_model(),
        "host_threads": os.cpu_count(),
    }


def _p10_p90(xs) -> list:
    """10th and 90th percentiles of a list of timings, rounded."""
    return [round(float(np.percentile(xs, 10)), 3), round(float(np.percentile(xs, 90)), 3)]


def _cpu_model() -> str:
    """lscpu's "Model name" (else /proc/cpuinfo's), as printed, with the x86
    family, model and stepping numbers (a virtualised host may print only
    the brand)."""
    import subprocess

    name = "unknown"
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                name = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    ids = {}
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                key, _, val = line.partition(":")
                key = key.strip()
                if key in ("model name", "cpu family", "model", "stepping") and key not in ids:
                    ids[key] = val.strip()
                if not line.strip() and ids:
                    break  # first processor only
    except OSError:
        pass
    if name == "unknown":
        name = ids.get("model name", "unknown")
    if "cpu family" in ids:
        name += f" (family {ids['cpu family']}, model {ids.get('model', '?')}, stepping {ids.get('stepping', '?')})"
    return name


# ---------------------------------------------------------------------------
# rocprofv3 summaries (run on CSV output: --output-format csv)
# ---------------------------------------------------------------------------

def _short_kernel(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    for pre in ("ugp::",):
        name = name.replace(pre, "")
    cut = name.find("(")
    return name[:cut] if cut > 0 else name


def summarize_trace(stats_csv: str) -> str:
    """Per-kernel durations from rocprofv3 --kernel-trace --stats (kernel_stats.csv)."""
    import csv

    rows = list(csv.DictReader(open(stats_csv, encoding="utf-8")))
    out = [f"{'kernel':44s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total%':>7s}"]
    for r in rows:
        out.append(f"{_short_kernel(r['Name'])[:44]:44s} {int(r['Calls']):6d} {float(r['AverageNs'])/1e3:9.2f} "
                   f"{float(r['MinNs'])/1e3:9.2f} {float(r['MaxNs'])/1e3:9.2f} {float(r['Percentage']):7.2f}")
    return "\n".join(out)


def _counter_means(csv_path: str, counter: str) -> dict:
    import csv

    acc: dict = {}
    for r in csv.DictReader(open(csv_path, encoding="utf-8")):
        if r.get("Counter_Name") != counter:
            continue
        k = _short_kernel(r["Kernel_Name"])
        acc.setdefault(k, []).append(float(r["Counter_Value"]))
    return acc


def summarize_counters(fetch_csv: str, write_csv: str, copy_bytes: int = 256 << 20) -> tuple[str, dict]:
    """Fabric bytes per dispatch from FETCH_SIZE / WRITE_SIZE (KiB), each scaled by
    what the same counter reads for the largest device copy (copy_bytes read
    and written) in the same run -- the reference copy of bench.py
    --copy-reference, which then skips its other copies."""
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    copy_key = next((k for k in fetch if "copyBuffer" in k), None)
    if copy_key is None:
        raise SystemExit("no copy kernel in the counter run (use --copy-reference)")
    f_scale = copy_bytes / (max(fetch[copy_key]) * 1024.0)
    w_scale = copy_bytes / (max(write[copy_key]) * 1024.0)
    lines = [f"copy reference: {copy_bytes} B read+written; FETCH_SIZE reads {max(fetch[copy_key]):.1f} KiB "
             f"(scale {f_scale:.3f}), WRITE_SIZE reads {max(write[copy_key]):.1f} KiB (scale {w_scale:.3f})",
             f"{'kernel':44s} {'dispatches':>10s} {'fetch_KiB':>11s} {'write_KiB':>11s} {'scaled_MB':>10s}"]
    traffic = {}
    for k in sorted(set(fetch) & set(write)):
        if "copyBuffer" in k:
            continue
        fk = sum(fetch[k]) / len(fetch[k])
        wk = sum(write[k]) / len(write[k])
        b = fk * 1024.0 * f_scale + wk * 1024.0 * w_scale
        traffic[k] = (b, len(fetch[k]))
        lines.append(f"{k[:44]:44s} {len(fetch[k]):10d} {fk:11.1f} {wk:11.1f} {b / 1e6:10.2f}")
    return "\n".join(lines), traffic


# kernel symbol -> stage name, for the traffic file
KERNEL_STAGE = {
    "staged_keys_kernel": "chunk_sort", "staged_cells_kernel": "tile_sort",
    "bucket_fine_count_kernel": "tile_scan", "bucket_colscan_kernel": "tile_scan", "bucket_rebucket_kernel": "rebucket",
    "clear_kernel": "clear", "count_kernel": "count", "scan_kernel": "scan",
    "scatter_kernel": "scatter", "gather_kernel": "gather", "fix_cells_kernel": "stable_sort",
}


def write_traffic_file(traffic: dict, path: str, command: str) -> None:
    with open(path, "w", encoding="utf-8") as f:
        f.write("# Measured fabric traffic per dispatch (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE: bytes between\n")
        f.write("# the L2 caches and the Infinity Fabric, Infinity Cache hits included),\n")
        f.write("# each counter scaled by its reading for a 256 MiB device copy in the same run.\n")
        f.write(f"# command: {command}\n")
        f.write(f"source_sha256_16: {source_digest()}\n")
        # per stage, the most-dispatched variant (the headline's; the
        # diagnostic and Morton variants run a few times beside it)
        # variant of each kernel; a stage of two kernels sums them. The
        # chunk kernel is the bucketed path's coarse_sort when bucket
        # kernels ran beside it
        bucketed = any(k.startswith("bucket_") for k in traffic)
        best = {}
        for k, (b, dispatches) in traffic.items():
            base = k.split("<")[0]
            if base not in KERNEL_STAGE:
                continue
            if base not in best or dispatches > best[base][1]:
                best[base] = (b, dispatches)
        per_stage = {}
        for base, (b, _) in best.items():
            stage = KERNEL_STAGE[base]
            if stage == "chunk_sort" and bucketed:
                stage = "coarse_sort"
            per_stage[stage] = per_stage.get(stage, 0.0) + b
        for stage, b in per_stage.items():
            f.write(f"{stage}_bytes_per_dispatch: {b:.0f}\n")


def candidate_pairs(conteos: np.ndarray, dims) -> int:
    """Distance evaluations of one 27-cell neighbour pass, from the linear
    histogram: every particle meets every particle of the (in-grid) 27 cells
    around its cell except itself."""
    nx, ny, nz = (int(v) for v in dims)
    c = conteos.astype(np.int64).reshape(nz, ny, nx)
    pad = np.pad(c, 1)
    box = np.zeros_like(c)
    for dz in range(3):
        for dy in range(3):
            for dx in range(3):
                box += pad[dz:dz + nz, dy:dy + ny, dx:dx + nx]
    return int((c * box).sum() - c.sum())


def neighbor_bench(ugp, torch, dev, evict, stream, reps: int = 5) -> dict:
    """27-cell neighbour count on the SPH-like workload: original order
    through ordenado (the indirection) vs the build's reordered records, with
    linear and Morton cell keys. Cold: caches evicted before each timing."""
    import workloads

    wl = workloads.make_sph_like()
    n, dims = wl.n, [int(v) for v in wl.dims]
    origin, h = [float(v) for v in wl.origin], float(wl.cell_size)
    radius = workloads.SPH_RADIUS_FRACTION * h
    parts = torch.from_numpy(wl.particles).to(dev)
    out = torch.empty(n, dtype=torch.int32, device=dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            evict()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            t.append(1e3 * e0.elapsed_time(e1))
        return statistics.median(t)

    res = {"workload": f"{n:,} uniform particles on {dims[0]}^3 cells (30.5 per cell), radius "
                       f"{workloads.SPH_RADIUS_FRACTION} cell",
           "radius": radius}
    lin = ugp.grid_build(parts, origin, h, dims)
    mor = ugp.grid_build(parts, origin, h, dims, morton=True)
    torch.cuda.synchronize()
    pairs = candidate_pairs(ugp.as_u32_numpy(lin.conteos), dims)
    res["candidate_pairs"] = pairs
    res["build_us"] = timed(lambda: ugp.grid_build(parts, origin, h, dims, out=lin))
    runs = {
        "indirect_linear": lambda: ugp.neighbor_count(parts, origin, h, dims, lin.inicios, lin.ordenado, radius, out=out),
        "reordered_linear": lambda: ugp.neighbor_count(lin.reordered, origin, h, dims, lin.inicios, None, radius, out=out),
        "indirect_morton": lambda: ugp.neighbor_count(parts, origin, h, dims, mor.inicios, mor.ordenado, radius,
                                                      morton=True, out=out),
        "reordered_morton": lambda: ugp.neighbor_count(mor.reordered, origin, h, dims, mor.inicios, None, radius,
                                                       morton=True, out=out),
    }
    for name, fn in runs.items():
        us = timed(fn)
        res[name] = {"us": round(us, 2), "pairs_per_s": pairs / (us * 1e-6)}
    res["mean_neighbors"] = float(ugp.as_u32_numpy(out).mean())
    res["speedup_reordered_vs_indirect"] = res["indirect_linear"]["us"] / res["reordered_linear"]["us"]
    res["speedup_morton_vs_linear_reordered"] = res["reordered_linear"]["us"] / res["reordered_morton"]["us"]
    res["note"] = ("one thread per query, queries taken in cell order; pairs = distance evaluations "
                   "(27-cell candidates, self excluded); the reordered runs read the build's cell-ordered "
                   "records, the indirect ones read the original array through ordenado")
    return res


def other_workloads_bench(ugp, torch, dev, evict, stream, steps: int = 20, warmup: int = 3) -> dict:
    """The other workloads of the build, each timed like the headline: warm-up
    builds, then `steps` cold builds (the same 1 GiB eviction before each,
    outside the per-build events), median with p10/p90. The method-level byte
    model (116 N + 16 C + 4) gives each its fraction of the 8 TB/s peak."""
    import workloads

    res = {}
    for name, mode in (("tiny", "atomic"), ("sparse", "atomic"), ("contention", "atomic"),
                       ("contention", "stable"), ("large", "atomic")):
        wl = workloads.make_config(name)
        dims = [int(v) for v in wl.dims]
        origin, h = [float(v) for v in wl.origin], float(wl.cell_size)
        stable = mode == "stable"
        parts = torch.from_numpy(wl.particles).to(dev)
        out, ws = ugp.alloc_outputs(wl.n, dims, dev, ugp.FLAG_STABLE if stable else 0)

        def build():
            ugp.grid_build(parts, origin, h, dims, stable=stable, out=out, workspace=ws)

        for _ in range(warmup):
            build()
        torch.cuda.synchronize()
        ini = ugp.as_u32_numpy(out.inicios)
        if int(ini[-1]) != wl.n:
            raise RuntimeError(f"{name}: inicios[C] != N after the warm-up builds")
        t = []
        for _ in range(steps):
            evict()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            build()
            e1.record(stream)
            torch.cuda.synchronize()
            t.append(1e3 * e0.elapsed_time(e1))
        med = statistics.median(t)
        model = 116 * wl.n + 16 * wl.cells + 4
        res[f"{name}_{mode}"] = {
            "workload": WORKLOAD_NAMES[name], "mode": mode, "us": round(med, 2), "us_p10_p90": _p10_p90(t),
            "particles_per_s": wl.n / (med * 1e-6), "hbm_frac_e2e": model / (med * 1e-6) / (HBM_PEAK_GBS * 1e9)}
        del parts, out, ws
        torch.cuda.empty_cache()
    res["note"] = ("cold builds (1 GiB read-only eviction before each, outside the per-build events), median of "
                   f"{steps} after {warmup} warm-up builds; hbm_frac_e2e from the byte model 116 N + 16 C + 4")
    return res


def reorder_policy_bench(ugp, torch, dev, evict, stream, reps: int = 5) -> dict:
    """Reorder policies of the reorder page on MI355X: (a) hot kinematics and
    cold appearance (32 bytes each) gathered with one index in one kernel vs
    two single-array gathers; (b) on the SPH-like workload, the per-frame
    cost of reordering every frame vs building only the index and querying
    neighbours through ordenado on an array reordered some frames ago."""
    import workloads

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            evict()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            t.append(1e3 * e0.elapsed_time(e1))
        return statistics.median(t)

    res = {}
    wl = workloads.make_config("baseline")
    n = wl.n
    hot = torch.from_numpy(wl.particles).to(dev)
    cold = torch.rand((n, 8), device=dev)
    idx = ugp.grid_build(hot, wl.origin.tolist(), float(wl.cell_size), wl.dims.tolist(), index_only=True).ordenado
    outs = [torch.empty_like(hot), torch.empty_like(cold)]
    one = timed(lambda: ugp.reorder_arrays(idx, [hot, cold], outs=outs))
    two = timed(lambda: (ugp.reorder(hot, idx, out=outs[0]), ugp.reorder(cold, idx, out=outs[1])))
    alg = 4 * n + 2 * 64 * n  # index once; each array 32 B read (gathered) + 32 B written
    res["hot_cold_split"] = {"n": n, "one_kernel_us": round(one, 2), "two_kernels_us": round(two, 2),
                             "one_kernel_GBps": round(alg / (one * 1e3), 1),
                             "note": "1M particles, two 32-byte arrays, the build's ordenado as the index"}

    wl = workloads.make_sph_like()
    n, dims = wl.n, [int(v) for v in wl.dims]
    origin, h = [float(v) for v in wl.origin], float(wl.cell_size)
    radius = workloads.SPH_RADIUS_FRACTION * h
    parts = torch.from_numpy(wl.particles).to(dev)
    full = ugp.grid_build(parts, origin, h, dims)
    state = full.reordered.clone()
    gen = torch.Generator(device=dev).manual_seed(7)
    frames = {}
    counts = torch.empty(n, dtype=torch.int32, device=dev)
    idx_out, idx_ws = ugp.alloc_outputs(n, dims, dev, ugp.FLAG_INDEX_ONLY)
    for age in range(1, 9):  # frames since the last reorder; particles move 0.05 cell (rms, per axis) a frame
        state[:, :3] += torch.randn((n, 3), device=dev, generator=gen) * (0.05 * h)
        if age in (1, 4, 8):
            b_us = timed(lambda: ugp.grid_build(state, origin, h, dims, index_only=True, out=idx_out, workspace=idx_ws))
            q_us = timed(lambda: ugp.neighbor_count(state, origin, h, dims, idx_out.inicios, idx_out.ordenado, radius,
                                                    out=counts))
            frames[f"age_{age}"] = {"index_only_build_us": round(b_us, 2), "query_through_ordenado_us": round(q_us, 2)}
    full_out, full_ws = ugp.alloc_outputs(n, dims, dev, 0)
    fb_us = timed(lambda: ugp.grid_build(state, origin, h, dims, out=full_out, workspace=full_ws))
    fq_us = timed(lambda: ugp.neighbor_count(full_out.reordered, origin, h, dims, full_out.inicios, None, radius,
                                             out=counts))
    res["every_n_frames"] = {
        "workload": "SPH-like, 1M particles on 32^3, radius 0.87 cell; 0.05 cell of motion per frame",
        "reorder_every_frame": {"build_us": round(fb_us, 2), "query_reordered_us": round(fq_us, 2),
                                "frame_us": round(fb_us + fq_us, 2)},
        "index_only_frames": frames,
    }
    return res


VALU_PEAK_OPS = 256 * 64 * 2.4e9  # lane-operations/s: 256 CUs x 64 lanes x 2.4 GHz (no packed fp32)
PAIR_OPS = 10  # VALU operations per candidate pair: 3 sub, 3 mul, 2 add, compare, count


def _oracle_time(fn, budget_s: float = 2.0) -> float:
    times = []
    t_end = time.perf_counter() + budget_s
    while True:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() >= t_end or len(times) >= 5:
            break
    return statistics.median(times)


def next_rows_summary(result: dict, wl, with_oracle: bool) -> dict:
    """Each row built past the four page steps, measured against its kernel's
    roofline with the oracle timed beside it (single-threaded, bounded)."""
    import workloads

    n, cells = wl.n, wl.cells
    step_us = result["ms_per_step"] * 1e3
    b_model = 116 * n + 16 * cells + 4
    rows = {}
    dv = result["diag_variant"]
    diag_gbs = 4 * cells / (dv["cell_diag_us"] * 1e3)
    rows["overflow_diagnostics"] = {
        "gpu": {"fused_step_us": round(dv["ms_per_step"] * 1e3, 2),
                "fused_overhead_us": round(dv["ms_per_step"] * 1e3 - step_us, 2),
                "standalone_us": dv["cell_diag_us"]},
        "roofline": {"kernel": "cell_diag_kernel<512> (standalone, over conteos)", "bound": "hbm", "achieved": round(diag_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": diag_gbs / HBM_PEAK_GBS},
    }
    mv = result["morton_variant"]
    mor_gbs = b_model / (mv["ms_per_step"] * 1e6)
    rows["morton_keys"] = {
        "gpu": {"step_us": round(mv["ms_per_step"] * 1e3, 2), "linear_step_us": round(step_us, 2)},
        "roofline": {"kernel": "whole build, Morton keys (byte model 116 N + 16 C + 4)", "bound": "hbm",
                     "achieved": round(mor_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": mor_gbs / HBM_PEAK_GBS},
    }
    nq = result.get("neighbor_query")
    if nq:
        best = nq["reordered_linear"]
        ops = best["pairs_per_s"] * PAIR_OPS
        rows["neighbor_query"] = {
            "gpu": {k: nq[k]["us"] for k in ("indirect_linear", "reordered_linear", "indirect_morton", "reordered_morton")},
            "roofline": {"kernel": "neighbor_count_kernel (reordered records, linear keys)", "bound": "alu",
                         "achieved": round(ops / 1e12, 2), "peak": round(VALU_PEAK_OPS / 1e12, 2),
                         "unit": "T lane-ops/s", "frac": ops / VALU_PEAK_OPS,
                         "note": f"{PAIR_OPS} VALU operations per candidate pair; peak = 256 CUs x 64 lanes x 2.4 GHz"},
        }
    rp = result.get("reorder_policy")
    if rp:
        hc = rp["hot_cold_split"]
        rows["multi_array_reorder"] = {
            "gpu": {"one_kernel_us": hc["one_kernel_us"], "two_kernels_us": hc["two_kernels_us"]},
            "roofline": {"kernel": "gather_arrays_kernel (two 32-byte arrays)", "bound": "hbm",
                         "achieved": hc["one_kernel_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": hc["one_kernel_GBps"] / HBM_PEAK_GBS},
        }
    if not with_oracle:
        return rows
    import oracle

    orc = oracle.load()
    ref = orc.grid_build(wl.particles, wl.origin, wl.cell_size, wl.dims)
    t = _oracle_time(lambda: orc.diag(ref.conteos, 64))
    rows["overflow_diagnostics"]["oracle"] = {"value": cells / t, "unit": "cells/s", "cores": 1,
                                              "sample": f"ugp_oracle_diag over the {cells} counts of the workload"}
    t = _oracle_time(lambda: orc.grid_build(wl.particles, wl.origin, wl.cell_size, wl.dims, morton=True))
    rows["morton_keys"]["oracle"] = {"value": n / t, "unit": "particles/s", "cores": 1,
                                     "sample": "full Morton-keyed build of the workload"}
    if nq:
        sph = workloads.make_sph_like()
        radius = workloads.SPH_RADIUS_FRACTION * float(sph.cell_size)
        idx = orc.grid_build(sph.particles, sph.origin, sph.cell_size, sph.dims)
        t = _oracle_time(lambda: orc.neighbor_count(sph.particles, sph.origin, sph.cell_size, sph.dims, radius,
                                                    index=idx), budget_s=1.0)
        rows["neighbor_query"]["oracle"] = {"value": nq["candidate_pairs"] / t, "unit": "candidate pairs/s",
                                            "cores": 1, "sample": "the whole SPH-like neighbour pass"}
    if rp:
        cold = np.ascontiguousarray(np.random.Generator(np.random.PCG64(1)).random((n, 8), dtype=np.float32))
        t = _oracle_time(lambda: (orc.gather(wl.particles, ref.ordenado), orc.gather(cold, ref.ordenado)))
        rows["multi_array_reorder"]["oracle"] = {"value": n / t, "unit": "particles/s", "cores": 1,
                                                 "sample": "two 32-byte arrays of the workload gathered by ordenado"}
    return rows


def main(argv=None) -> int:
    if argv is None and len(sys.argv) > 1 and sys.argv[1] == "summarize":
        return summarize_main(sys.argv[2:])
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="baseline", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--mode", default="atomic", choices=["atomic", "gather", "stable"])
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle timing (0 = skip)")
    ap.add_argument("--no-neighbors", action="store_true",
                    help="skip the neighbour-query, reorder-policy and other-workload sections")
    ap.add_argument("--presorted", action="store_true",
                    help="time the workload's records already in cell order (the build's own reordered "
                         "output of one untimed build), the secondary variant of the contention config")
    ap.add_argument("--copy-reference", action="store_true",
                    help="also run a 256 MiB device copy (counter calibration for rocprofv3 --pmc)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print("bench.py measures one GPU only: the index build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import uniform_grid_particle_amd as ugp
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    ugp.load_library()

    wl = workloads.make_config(args.workload)
    n, dims, cells = wl.n, [int(v) for v in wl.dims], wl.cells
    origin, h = [float(v) for v in wl.origin], float(wl.cell_size)
    flags = {"atomic": 0, "gather": ugp.FLAG_GATHER, "stable": ugp.FLAG_STABLE}[args.mode]
    parts = torch.from_numpy(wl.particles).to(dev)
    if args.presorted:
        # records in cell order: one untimed build's own reordered output (the
        # order inside a cell is that build's); the oracle timing below then
        # runs on the same records
        first = ugp.grid_build(parts, origin, h, dims)
        torch.cuda.synchronize()
        parts = first.reordered.clone()
        wl = workloads.Workload(wl.name + "_presorted", parts.cpu().numpy(), wl.origin, wl.cell_size, wl.dims)
        del first
    out, ws = ugp.alloc_outputs(n, dims, dev, flags)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB, read to evict caches

    def evict():
        torch.sum(flush)
    stream = torch.cuda.current_stream(dev)

    def build():
        ugp.grid_build(parts, origin, h, dims, stable=args.mode == "stable", gather=args.mode == "gather",
                       out=out, workspace=ws)

    for _ in range(args.warmup):
        build()
    torch.cuda.synchronize()
    # light self-check of the warm-up output (full parity lives in the tests)
    ini = ugp.as_u32_numpy(out.inicios)
    if int(ini[-1]) != n or int(ugp.as_u32_numpy(out.conteos).sum(dtype=np.uint64)) != n:
        print("bench self-check failed: inicios[C] or sum(conteos) != N", file=sys.stderr)
        return 1

    if args.copy_reference:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    # ---- headline: K cold steps, each bracketed by events ----
    K = args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for k in range(K):
        evict()
        starts[k].record(stream)
        build()
        ends[k].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = [starts[k].elapsed_time(ends[k]) for k in range(K)]
    # the median step (with p10/p90): a single step delayed by the host (the
    # GPU idles until the launch arrives) must not stand for the kernels
    ms_per_step = statistics.median(step_ms)
    ms_mean = sum(step_ms) / K

    # ---- achievable bandwidth on this device: cold device-to-device copies,
    # one of 1 GiB moved (512 MiB read + 512 MiB written) and one moving the
    # same number of bytes as the byte model of one step ----
    def copy_gbs(nbytes_moved: int) -> float:
        half = max(1, nbytes_moved // 2)
        src = torch.ones(half, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        t = []
        for _ in range(5):
            evict()
            c0 = torch.cuda.Event(enable_timing=True)
            c1 = torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            dst.copy_(src)
            c1.record(stream)
            torch.cuda.synchronize()
            t.append(c0.elapsed_time(c1))
        del src, dst
        return 2 * half / (statistics.median(t) * 1e-3) / 1e9

    if args.copy_reference:  # counter runs: the 256 MiB reference must stay the largest copy
        copy_big = copy_same = None
    else:
        copy_big = copy_gbs(1 << 30)
        copy_same = copy_gbs(116 * n + 16 * cells + 4)

    # ---- overflow-diagnostics variant (capacity 64): K cold builds with the
    # reduction folded into the build, then the standalone reduction over
    # the final conteos ----
    diag = torch.empty(2, dtype=torch.int32, device=dev)
    dstarts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    dends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for k in range(K):
        evict()
        dstarts[k].record(stream)
        ugp.grid_build_diag(parts, origin, h, dims, 64, diag=diag, stable=args.mode == "stable",
                            gather=args.mode == "gather", out=out, workspace=ws)
        dends[k].record(stream)
    torch.cuda.synchronize()
    diag_steps = [dstarts[k].elapsed_time(dends[k]) for k in range(K)]
    diag_ms = statistics.median(diag_steps)
    diag_val = [int(v) for v in ugp.as_u32_numpy(diag)]
    # standalone reduction, cold, timed by its kernel's own start and end;
    # then the same entry point over an empty histogram (one workgroup, no
    # loads), the fixed cost of any launch on this clock
    def diag_kernel_us(conteos):
        t = []
        for _ in range(K):
            evict()
            c0 = torch.cuda.Event(enable_timing=True)
            c1 = torch.cuda.Event(enable_timing=True)
            ugp.cell_diag_timed(conteos, 64, c0, c1, out=diag)
            torch.cuda.synchronize()
            t.append(1e3 * c0.elapsed_time(c1))
        return t
    cd = diag_kernel_us(out.conteos)
    cell_diag_us = statistics.median(cd)
    cd0 = diag_kernel_us(out.conteos[:0])

    # ---- Morton-keyed variant: K cold builds numbering cells along the Z curve ----
    mflags = flags | ugp.FLAG_MORTON
    mout, mws = ugp.alloc_outputs(n, dims, dev, mflags)
    mstarts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    mends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for k in range(K):
        evict()
        mstarts[k].record(stream)
        ugp.grid_build(parts, origin, h, dims, stable=args.mode == "stable", gather=args.mode == "gather",
                       morton=True, out=mout, workspace=mws)
        mends[k].record(stream)
    torch.cuda.synchronize()
    morton_steps = [mstarts[k].elapsed_time(mends[k]) for k in range(K)]
    morton_ms = statistics.median(morton_steps)
    del mout, mws

    # ---- warm: K back-to-back builds between one event pair ----
    w0 = torch.cuda.Event(enable_timing=True)
    w1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0.record(stream)
    for _ in range(K):
        build()
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / K

    # ---- per-stage: for every stage slot, K cold steps of the full build with
    # two events recorded around that slot inside the same C call ----
    names = ugp.stage_names(n, dims, flags)
    bytes_k = alg_bytes(n, cells, args.mode)
    stages = {}
    for st, name in enumerate(names):
        if name is None:
            continue
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        torch.cuda.synchronize()
        for k in range(K):
            evict()
            ugp.grid_build_timed(st, evs[k][0], evs[k][1], parts, origin, h, dims, out, ws, flags=flags)
        torch.cuda.synchronize()
        per = [1e3 * e0.elapsed_time(e1) for e0, e1 in evs]
        us = statistics.median(per)
        b = bytes_k.get(name)
        gbs = (b / (us * 1e3)) if (b and us > 0) else None
        stages[name] = {"slot": st, "us": round(us, 3), "us_p10_p90": _p10_p90(per), "alg_bytes": b,
                        "GBps": None if gbs is None else round(gbs, 1),
                        "frac_hbm": None if gbs is None else round(gbs / HBM_PEAK_GBS, 4)}

    b_total = 116 * n + 16 * cells + 4
    dominant = max((st for st in stages if stages[st]["GBps"] is not None), key=lambda st: stages[st]["us"])
    dom_us = stages[dominant]["us"]
    achieved = bytes_k[dominant] / (dom_us * 1e3)
    traffic = read_traffic(dominant)

    t_s = ms_per_step * 1e-3
    result = {
        "metric": METRIC,
        "value": n / t_s,
        "unit": "particles/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_NAMES[args.workload] + (" (records pre-sorted by cell)" if args.presorted else ""),
            "n_particles": n,
            "dims": dims,
            "cells": cells,
            "cell_size": h,
            "seed": wl.seed,
            "mode": args.mode,
            "timing": "cold: 1 GiB read-only cache eviction before each step, outside the per-step HIP events; "
                      "ms_per_step is the median of the K steps (mean, p10/p90 and worst step also reported)",
        },
        "hbm_frac_e2e": (b_total / t_s) / (HBM_PEAK_GBS * 1e9),
        "achievable_copy_GBps": None if copy_big is None else {
            "1GiB": round(copy_big, 1), "same_bytes": round(copy_same, 1),
            "note": "cold device-to-device copy, bytes read + written / time"},
        "frac_of_copy_e2e": None if copy_big is None else {
            "1GiB": (b_total / t_s) / (copy_big * 1e9), "same_bytes": (b_total / t_s) / (copy_same * 1e9)},
        "alg_bytes_per_step": b_total,
        "step_ms_median": statistics.median(step_ms),
        "step_ms_mean": ms_mean,
        "step_ms_worst": [max(step_ms), int(np.argmax(step_ms))],
        "step_ms_p10_p90": [float(np.percentile(step_ms, 10)), float(np.percentile(step_ms, 90))],
        "warm_ms_per_step": warm_ms,
        "morton_variant": {"ms_per_step": morton_ms, "ms_p10_p90": _p10_p90(morton_steps),
                           "keys": ugp.key_count(dims, mflags),
                           "note": "same cold protocol (median of K steps), cells numbered along the Z curve"},
        "diag_variant": {"capacity": 64, "ms_per_step": diag_ms, "ms_p10_p90": _p10_p90(diag_steps),
                         "max_per_cell_and_overflows": diag_val,
                         "note": "same cold protocol (median of K steps), overflow diagnostics folded into the build",
                         "cell_diag_us": round(cell_diag_us, 3), "cell_diag_us_p10_p90": _p10_p90(cd),
                         "cell_diag_empty_us": round(statistics.median(cd0), 3),
                         "cell_diag_timing": "kernel's own start and end events, cold; "
                                             "_empty_us: the same call over zero cells (launch and ticket only)",
                         "cell_diag_GBps": round(4 * cells / (cell_diag_us * 1e3), 1)},
        "warm_note": "back-to-back builds; the working set can stay in the 256 MiB Infinity Cache",
        "stages": stages,
        "stage_sum_us": round(sum(s["us"] for s in stages.values()), 3),
        "stage_note": "each stage timed inside a full cold build (one C call): a one-kernel stage by events at its "
                      "kernel's own start and end (hipExtLaunchKernel), other stages by events around the stage; "
                      "median of K builds per stage, p10/p90 beside it; GBps and frac_hbm use the kernel-I/O bytes "
                      "(alg_bytes: every array a kernel reads or writes, counted once for that kernel)",
        "wall_s_timed_loop": wall,
        "roofline": {
            "kernel": dominant,
            "kernel_us": round(dom_us, 3),
            "alg_bytes": bytes_k[dominant],
            "bytes_model": "kernel I/O: every array the kernel reads or writes, counted once (the build's own "
                           "intermediate arrays included); the method-level figure is hbm_frac_e2e",
            "timing": "cold: median over K cold builds of the kernel's own start-to-end time (events recorded by "
                      "the launch itself, hipExtLaunchKernel)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": None if achieved is None else achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "traffic_note": "fabric traffic per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE between L2 and the "
                            "Infinity Fabric, each scaled by its reading for a plain device copy; Infinity Cache "
                            "hits included), or null when the kernel sources changed since it was counted",
        },
    }
    if not args.no_neighbors:
        result["neighbor_query"] = neighbor_bench(ugp, torch, dev, evict, stream)
        result["reorder_policy"] = reorder_policy_bench(ugp, torch, dev, evict, stream)
        if args.workload == "baseline" and args.mode == "atomic" and not args.presorted:
            result["other_workloads"] = other_workloads_bench(ugp, torch, dev, evict, stream)
    result["next_rows"] = next_rows_summary(result, wl, with_oracle=args.cpu_budget > 0)
    if args.cpu_budget > 0 and int(os.environ.get("RANK", "0")) == 0:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


def summarize_main(argv) -> int:
    """python bench.py summarize trace STATS_CSV
       python bench.py summarize counters FETCH_CSV WRITE_CSV [--write-traffic PATH --command CMD]"""
    ap = argparse.ArgumentParser(prog="bench.py summarize")
    ap.add_argument("kind", choices=["trace", "counters"])
    ap.add_argument("files", nargs="+")
    ap.add_argument("--write-traffic")
    ap.add_argument("--command", default="")
    a = ap.parse_args(argv)
    if a.kind == "trace":
        print(summarize_trace(a.files[0]))
        return 0
    text, traffic = summarize_counters(a.files[0], a.files[1])
    print(text)
    if a.write_traffic:
        write_traffic_file(traffic, a.write_traffic, a.command)
    return 0


if __name__ == "__main__":
    sys.exit(main())
