"""Compile libsbd.so (all HIP sources under csrc/, gfx950) in-tree with hipcc,
and the benchmark's memory-ceiling kernels (ceiling/) into a library of their
own, libsbd_ceiling.so, which the delta library never links or loads."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libsbd.so")
CEILING_LIB = os.path.join(PKG, "libsbd_ceiling.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _compile(out, srcs, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _compile(LIB, sources(), verbose)
    _compile(CEILING_LIB, [os.path.join(PKG, "ceiling", "ceiling.hip")], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
