"""CPU tests: every oracle pin again, against a copy of the oracle built with
gcc's AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

The instrumented library is loaded in a child Python process with the ASan
runtime preloaded (the interpreter itself is not instrumented, so its own
allocations are not leak-checked). A heap or stack overrun, use after free,
signed overflow, misaligned access or out-of-range shift inside the oracle
aborts the child with the sanitizer's report, and the test fails with it.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]

# The child runs every pin of tests/pins.py on small inputs: the worked
# example, special positions and clamping, the binary32 model, brute-force
# slices, empty and degenerate grids, grid validation, Morton keys,
# neighbour counts, the diagnostics' closed form and the byte gather.
CHILD = r"""
import sys
sys.path.insert(0, ROOT)
import numpy as np
import oracle
import workloads as W
from tests import pins

orc = oracle.Oracle(LIB)
pins.pin_worked_example_scan(orc)
pins.pin_worked_example_pipeline(orc)
pins.pin_cell_centres_noncubic(orc)
pins.pin_special_positions(orc)
pins.pin_diag_closed_form(orc)
pins.pin_grid_validation(orc)
pins.pin_empty_and_degenerate(orc)
pins.pin_morton_textbook(orc)
pins.pin_morton_recursion_bijection(orc)
pins.pin_neighbors_lattice(orc)
pins.pin_gather_bytes(orc)
for wl in (W.make_config("tiny"), W.make_contention(20_000, 16, seed=3, hot=2_000, per_cluster=3_000, outside=1_000),
           W.make_uniform(5_000, 7, seed=11)):
    pins.pin_binary32_model(orc, wl)
    pins.pin_exact_floor_far_from_faces(orc, wl)
    pins.pin_library_reductions(orc, wl)
    pins.pin_brute_force_slices(orc, wl)
    pins.pin_morton_relabels_linear(orc, wl)
    r = orc.grid_build(wl.particles, wl.origin, wl.cell_size, wl.dims)
    pins.check_index_invariants(wl, r, stable=True)
    lo = np.asarray(wl.origin, np.float64)
    hi = lo + np.asarray(wl.dims, np.float64) * float(wl.cell_size)
    p = wl.particles[:, :3].astype(np.float64)
    inside = wl.particles[np.all((p >= lo) & (p < hi), axis=1)][:400]
    small = W.Workload(wl.name, np.ascontiguousarray(inside), wl.origin, wl.cell_size, wl.dims)
    h = float(wl.cell_size)
    pins.pin_neighbors_brute_force(orc, small, 0.9 * h)
    pins.pin_neighbors_brute_force(orc, small, 0.9 * h, morton=True)
print("SANITIZED PINS OK", flush=True)
"""


def _runtime(name: str) -> str | None:
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    lib = oracle.build(out=str(tmp_path / "libugp_oracle_sanitized.so"), extra=SANITIZE)
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "PYTHONPATH": ROOT,
    })
    script = f"ROOT = {ROOT!r}\nLIB = {lib!r}\n" + CHILD
    p = subprocess.run([sys.executable, "-c", script], env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=600)
    report = (p.stdout + p.stderr)[-6000:]
    assert p.returncode == 0, report
    assert "SANITIZED PINS OK" in p.stdout, report
    assert "runtime error" not in p.stderr, report
    assert "AddressSanitizer" not in p.stderr, report
