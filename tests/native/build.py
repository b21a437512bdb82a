"""Compile the native ABI smoke program against the in-tree libsbd.so."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "sparse_bf16_delta_amd")
BIN = os.path.join(HERE, "abi_smoke")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    # host code only; libsbd.so is found next to the package at run time
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "abi_smoke.cpp"),
           "-L", PKG, "-lsbd", f"-Wl,-rpath,{PKG}", "-Wl,-rpath,$ORIGIN/../../sparse_bf16_delta_amd",
           "-o", BIN + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(BIN + ".tmp", BIN)
    return BIN


if __name__ == "__main__":
    print(build(verbose=True))
