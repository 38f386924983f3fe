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


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def assembly(out: str) -> str:
    """Device assembly of the library, for inspection (gfx950 only)."""
    cmd = [HIPCC, *[f for f in FLAGS if f not in ("-shared", "-fPIC")], "-I", INCLUDE,
           "--cuda-device-only", "-S", SRC, "-o", out]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    if len(sys.argv) > 1:
        print(assembly(sys.argv[1]))
