"""Compile the HIP library (libugp.so) in-tree for gfx950 with hipcc."""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "ugp.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libugp.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3",
    "-std=c++17",
    "--offload-arch=gfx950",
    "-fPIC",
    "-shared",
    # no fast-math anywhere: the cell key needs the correctly rounded division
    "-fno-fast-math",
    "-ffp-contract=off",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def sources() -> list:
    """Every translation unit: the host code and C ABI (ugp.hip) and the tile
    kernel variants (tile_sort_*.hip), compiled in parallel."""
    d = os.path.dirname(SRC)
    return [SRC] + sorted(os.path.join(d, f) for f in os.listdir(d) if f.startswith("tile_sort_") and f.endswith(".hip"))


def build(verbose: bool = False) -> str:
    objs, procs = [], []
    for src in sources():
        obj = os.path.join(os.path.dirname(LIB), "_obj_" + os.path.basename(src) + ".o")
        cmd = [HIPCC, *[f for f in FLAGS if f != "-shared"], "-I", INCLUDE, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), cmd))
        objs.append(obj)
    failed = [cmd for p, cmd in procs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    for obj in objs:
        os.remove(obj)
    return LIB


def assembly(out: str) -> str:
    """Device assembly of every translation unit, concatenated (gfx950 only),
    for inspection."""
    parts = []
    for src in sources():
        part = out + "." + os.path.basename(src) + ".s"
        cmd = [HIPCC, *[f for f in FLAGS if f not in ("-shared", "-fPIC")], "-I", INCLUDE,
               "--cuda-device-only", "-S", src, "-o", part]
        parts.append((subprocess.Popen(cmd), part))
    with open(out, "w") as f:
        for p, part in parts:
            if p.wait() != 0:
                raise subprocess.CalledProcessError(1, part)
            with open(part) as g:
                f.write(g.read())
            os.remove(part)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    if len(sys.argv) > 1:
        print(assembly(sys.argv[1]))
