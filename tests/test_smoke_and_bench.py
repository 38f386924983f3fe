"""The benchmark's output contract: one JSON line carrying the metric, the
roofline of the dominant kernel and the CPU baseline, for one GPU only."""

from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU only" in r.stderr


@pytest.mark.gpu
def test_bench_json_line():
    print("[bench] short default run", flush=True)
    r = subprocess.run([sys.executable, BENCH, "--steps", "3", "--warmup", "1", "--cpu-budget", "1", "--no-neighbors"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [line for line in r.stdout.splitlines() if line.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "particles/s" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["config"]["workload"].startswith("Baseline")
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert abs(d["value"] - 1_000_000 / (d["ms_per_step"] * 1e-3)) <= 1e-6 * d["value"]
    # the four steps' byte model at 1M particles on 128^3 cells: 116 N + 16 C + 4
    assert d["alg_bytes_per_step"] == 149_554_436
    rf = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in rf, key
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0.0 < rf["frac"] < 1.0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    cb = d["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in cb, key
    assert cb["kind"] == "oracle" and cb["cores"] == 1 and cb["value"] > 0


@pytest.mark.gpu
def test_other_workloads_section():
    """The default run's timings of the other workloads: one entry per
    workload and mode, each a positive median with its spread."""
    print("[bench] other workloads, 2 cold builds each", flush=True)
    sys.path.insert(0, ROOT)
    import torch

    import bench
    import uniform_grid_particle_amd as ugp

    ugp.load_library()
    dev = torch.device("cuda:0")
    flush = torch.ones(1 << 26, dtype=torch.float32, device=dev)
    res = bench.other_workloads_bench(ugp, torch, dev, lambda: torch.sum(flush), torch.cuda.current_stream(dev),
                                      steps=2, warmup=1)
    keys = {"tiny_atomic", "sparse_atomic", "contention_atomic", "contention_stable", "large_atomic"}
    assert keys <= set(res), sorted(res)
    for k in keys:
        v = res[k]
        assert v["us"] > 0 and 0 < v["hbm_frac_e2e"] < 1 and len(v["us_p10_p90"]) == 2, (k, v)


@pytest.mark.gpu
def test_smoke_entry_point():
    sys.path.insert(0, ROOT)
    import __graft_entry__

    __graft_entry__.smoke()
