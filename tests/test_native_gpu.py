"""The C ABI from native code: a C++ program (tests/native/abi_smoke.cpp)
linked against libsbd.so, with no Python in its process, runs diff, apply,
XOR and the batched pair on the GPU and checks them by their defining
properties.  The program is compiled by the build step, not here."""
import os
import subprocess

import pytest
import torch

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "abi_smoke")


def test_native_program_uses_the_c_abi():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(BIN), "tests/native/abi_smoke is missing: run the build step first"
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "abi_smoke ok" in r.stdout
