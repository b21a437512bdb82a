"""The C-ABI boundary without a GPU: the library loads, exports every entry
point include/sbd.h declares, sizes workspaces, and rejects bad arguments
before touching the device.  The Python layer rejects bad tensors."""
import ctypes
import os
import re

import pytest
import torch

from conftest import ROOT

import sparse_bf16_delta_amd as sbd
from sparse_bf16_delta_amd import _abi

HEADER = os.path.join(ROOT, "include", "sbd.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_path():
    names = header_functions()
    for want in ("delta_workspace_size", "delta_diff", "delta_diff_many", "delta_apply",
                 "delta_apply_many", "xor_mask", "xor_apply", "delta_last_error"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = _abi.load()
    for name in header_functions():
        assert hasattr(lib, name), name
    assert set(header_functions()) == set(_abi.SIGNATURES)


def test_single_hip_runtime_in_process():
    _abi.load()
    maps = open("/proc/self/maps").read()
    paths = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(paths) == 1, paths


def test_workspace_size():
    lib = _abi.load()
    assert lib.delta_workspace_size(-1, 1) == 0
    assert lib.delta_workspace_size(1, -1) == 0
    a = lib.delta_workspace_size(1 << 20, 1)
    b = lib.delta_workspace_size(1 << 30, 1)
    c = lib.delta_workspace_size(1 << 30, 300)
    assert 0 < a < b < c
    # per 32768-element tile: a 2 KB staging slot and 32 KB of staging arena
    # (its worst case: 8192 staged changes), count, prefix, dense-list entry,
    # a 32-byte descriptor and an 8-byte arena position; each extra parameter
    # may add a partial tile and a 32-byte table entry
    per_tile = 2048 + 32768 + 4 + 4 + 4 + 32 + 8
    tiles = (1 << 30) // 32768
    assert b >= per_tile * tiles
    # no more than the layout needs: the slots start past a 1 MB boundary
    assert b <= per_tile * (tiles + 2) + 4096 * 4 + (1 << 20) + 9472
    assert c - b >= 299 * per_tile - (1 << 20)  # less what the slot alignment absorbs


def _err(lib):
    return lib.delta_last_error().decode()


def test_argument_errors_return_before_any_launch():
    lib = _abi.load()
    one = ctypes.c_void_p(16)  # never dereferenced: every call below is rejected first
    assert lib.delta_diff(one, one, -1, one, one, 0, one, one, 1 << 20, None) == _abi.DELTA_E_INVALID
    assert "n=-1" in _err(lib)
    assert lib.delta_diff(one, one, 1 << 31, one, one, 0, one, one, 1 << 40, None) == _abi.DELTA_E_RANGE
    assert "int32" in _err(lib)
    assert lib.delta_diff(one, one, 10, one, one, 0, None, one, 1 << 20, None) == _abi.DELTA_E_INVALID
    assert lib.delta_diff(None, one, 10, one, one, 5, one, one, 1 << 20, None) == _abi.DELTA_E_INVALID
    assert lib.delta_diff(one, one, 10, None, one, 5, one, one, 1 << 20, None) == _abi.DELTA_E_INVALID
    assert lib.delta_diff(one, one, 10, one, one, -1, one, one, 1 << 20, None) == _abi.DELTA_E_INVALID
    assert lib.delta_diff(one, one, 10, one, one, 5, one, one, 16, None) == _abi.DELTA_E_WORKSPACE
    assert lib.delta_diff(one, one, 10, one, one, 5, one, None, 1 << 20, None) == _abi.DELTA_E_WORKSPACE
    ptrs = (ctypes.c_void_p * 2)(16, 16)
    big = (ctypes.c_int64 * 2)(10, 1 << 31)
    neg = (ctypes.c_int64 * 2)(10, -3)
    assert lib.delta_diff_many(2, ptrs, ptrs, big, one, one, 10, one, one, one, 1 << 40,
                               None) == _abi.DELTA_E_RANGE
    assert "numels[1]" in _err(lib)
    assert lib.delta_diff_many(2, ptrs, ptrs, neg, one, one, 10, one, one, one, 1 << 40,
                               None) == _abi.DELTA_E_INVALID
    assert lib.delta_diff_many(-1, ptrs, ptrs, neg, one, one, 10, one, one, one, 1 << 40,
                               None) == _abi.DELTA_E_INVALID
    assert lib.delta_diff_many(2, ptrs, ptrs, big, one, one, 10, one, None, one, 1 << 40,
                               None) == _abi.DELTA_E_INVALID
    nul = (ctypes.c_void_p * 2)(16, None)
    ok2 = (ctypes.c_int64 * 2)(10, 10)
    assert lib.delta_diff_many(2, nul, ptrs, ok2, one, one, 10, one, one, one, 1 << 40,
                               None) == _abi.DELTA_E_INVALID
    assert lib.delta_diff_many(2, ptrs, ptrs, ok2, one, one, 10, one, one, one, 64,
                               None) == _abi.DELTA_E_WORKSPACE
    # more than 2^23 tiles of 32768 elements in one call
    k = 129
    kp = (ctypes.c_void_p * k)(*([16] * k))
    kn = (ctypes.c_int64 * k)(*([(1 << 31) - 1] * k))
    assert lib.delta_diff_many(k, kp, kp, kn, one, one, 10, one, one, one, 1 << 40,
                               None) == _abi.DELTA_E_RANGE
    assert "tiles" in _err(lib)
    assert lib.delta_apply(one, -1, one, one, 3, None) == _abi.DELTA_E_INVALID
    assert lib.delta_apply(one, 1 << 31, one, one, 3, None) == _abi.DELTA_E_RANGE
    assert lib.delta_apply(None, 10, one, one, 3, None) == _abi.DELTA_E_INVALID
    assert lib.delta_apply_checked(one, 10, one, one, 3, None, None) == _abi.DELTA_E_INVALID
    assert lib.delta_apply_checked(one, -1, one, one, 3, one, None) == _abi.DELTA_E_INVALID
    assert lib.delta_apply_many(2, ptrs, big, one, one, one, 5, None, one, 1 << 20,
                                None) == _abi.DELTA_E_RANGE
    assert lib.delta_apply_many(2, ptrs, ok2, one, one, one, 5, None, one, 8,
                                None) == _abi.DELTA_E_WORKSPACE
    assert lib.delta_apply_many(2, ptrs, ok2, one, one, None, 5, None, one, 1 << 20,
                                None) == _abi.DELTA_E_INVALID
    # a workspace that is large enough but not 256-byte aligned
    odd = ctypes.c_void_p(256 + 16)
    assert lib.delta_diff(one, one, 10, one, one, 5, one, odd, 1 << 40, None) == _abi.DELTA_E_WORKSPACE
    assert "256-byte" in _err(lib)
    assert lib.delta_diff_many(2, ptrs, ptrs, ok2, one, one, 10, one, one, odd, 1 << 40,
                               None) == _abi.DELTA_E_WORKSPACE
    assert "256-byte" in _err(lib)
    assert lib.delta_apply_many(2, ptrs, ok2, one, one, one, 5, None, odd, 1 << 40,
                                None) == _abi.DELTA_E_WORKSPACE
    assert "256-byte" in _err(lib)
    assert lib.xor_mask(one, None, one, 5, None) == _abi.DELTA_E_INVALID
    assert lib.xor_mask(one, one, one, -5, None) == _abi.DELTA_E_INVALID
    assert lib.xor_apply(None, one, 5, None) == _abi.DELTA_E_INVALID
    # counts above 2^62 (e.g. INT64_MAX as "no limit") are refused, not rounded
    # into an overflowing grid
    top = (1 << 63) - 1
    assert lib.delta_apply_many(2, ptrs, ok2, one, one, one, top, None, one, 1 << 20,
                                None) == _abi.DELTA_E_RANGE
    assert "above 2^62" in _err(lib)
    assert lib.delta_apply(one, 10, one, one, top, None) == _abi.DELTA_E_RANGE
    assert lib.xor_mask(one, one, one, top, None) == _abi.DELTA_E_RANGE
    assert lib.xor_apply(one, one, top, None) == _abi.DELTA_E_RANGE
    assert lib.xor_apply_streamed(one, one, top, 64, one, 1 << 40, None, None) == _abi.DELTA_E_RANGE
    assert lib.delta_wire_checksum(one, top, one, 4, one, None) == _abi.DELTA_E_RANGE
    assert lib.delta_wire_hash(one, 4, one, top, one, None) == _abi.DELTA_E_RANGE
    w1 = (ctypes.c_int64 * 1)(10)
    assert lib.delta_wire_encode(1, w1, one, one, top, one, 10, one, one, 1 << 30,
                                 None) == _abi.DELTA_E_RANGE
    assert lib.delta_wire_decode(1, w1, one, top, one, one, 5, one, None, one, 1 << 30,
                                 None) == _abi.DELTA_E_RANGE
    assert lib.delta_wire_encode_blocked(1, w1, one, one, top, one, 64, one, 1 << 30,
                                         None) == _abi.DELTA_E_RANGE
    assert lib.delta_wire_decode_blocked(1, w1, one, 64, one, top, one, None, one, 1 << 30,
                                         None) == _abi.DELTA_E_RANGE


def test_error_message_is_per_thread():
    """delta_last_error describes the calling thread's last failure: threads
    failing at the same time with different arguments (ctypes releases the
    GIL during each call) each read back their own message."""
    import threading

    lib = _abi.load()
    one = ctypes.c_void_p(16)  # never dereferenced: every call is rejected first
    barrier = threading.Barrier(4)
    bad = []

    def worker(k):
        n = -(1000 + k)
        barrier.wait()
        for _ in range(2000):
            if lib.delta_diff(one, one, n, one, one, 0, one, one, 1 << 20, None) != _abi.DELTA_E_INVALID:
                bad.append((k, "status"))
                return
            if f"n={n}" not in lib.delta_last_error().decode():
                bad.append((k, lib.delta_last_error().decode()))
                return

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not bad, bad


def test_python_layer_rejects_bad_tensors():
    cpu = torch.zeros(8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        sbd.diff(cpu, cpu)
    with pytest.raises(ValueError, match="dtype"):
        sbd.diff(torch.zeros(8, dtype=torch.float32), torch.zeros(8, dtype=torch.float32))
    with pytest.raises(TypeError):
        sbd.xor_mask([1, 2], [1, 2])
    with pytest.raises(ValueError):
        sbd.diff_many([], [])


def test_binding_makes_the_tensors_device_current():
    """The library works on the calling thread's current device, so every
    wrapper that calls it runs under its tensors' device; host-only
    arguments leave the current device alone."""
    from sparse_bf16_delta_amd import ops

    for name in ("diff", "diff_many", "apply_", "apply_many_", "apply_many_host_",
                 "apply_streamed_", "xor_apply_streamed_", "xor_mask", "xor_apply_",
                 "wire_encode", "wire_decode", "wire_encode_blocked", "wire_decode_blocked",
                 "wire_hashes", "wire_checksum"):
        assert hasattr(getattr(ops, name), "__wrapped__"), name
    cpu = torch.zeros(4, dtype=torch.bfloat16)
    assert ops._device_of([cpu, [cpu], (), 3, None]) is None
    src = open(os.path.join(ROOT, "sparse_bf16_delta_amd", "plan.py")).read()
    assert src.count("with torch.cuda.device(") == 3  # the three plans' run()


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(_abi, "_lib", None)
    monkeypatch.setattr(_abi, "LIB_PATH", os.path.join(ROOT, "no_such_libsbd.so"))
    with pytest.raises(ImportError, match="no CPU fallback"):
        _abi.load()


def test_product_path_does_not_touch_the_oracle():
    """The package never imports, links or opens anything under oracle/."""
    pkg = os.path.join(ROOT, "sparse_bf16_delta_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f
    assert "oracle" not in open(HEADER).read().lower()


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 (or a launcher's WORLD_SIZE
    above 1) exits with a message before touching a device."""
    import subprocess
    import sys

    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
    env["WORLD_SIZE"] = "8"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")],
                       capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 2 and "WORLD_SIZE=8" in r.stderr


def _declaration(name):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    m = re.search(r"\b" + name + r"\s*\(([^)]*)\)\s*;", text)
    assert m, name
    params = [" ".join(p.replace("*", " * ").split()) for p in m.group(1).split(",")]
    # drop the parameter names, keep the types
    return [p.rsplit(" ", 1)[0] if p != "void" else p for p in params]


def test_core_signatures_are_the_boundary_contract():
    """The core calls keep the argument lists of the boundary contract: the
    sparse delta (int32 indices, bf16 bits, device count, workspace), the
    in-place apply with a host entry count, and the XOR pair.  The stream is
    a hipStream_t passed as void* so that the header needs no HIP include."""
    u16c, u16 = "const uint16_t *", "uint16_t *"
    assert _declaration("delta_workspace_size") == ["int64_t", "int32_t"]
    assert _declaration("delta_diff") == [u16c, u16c, "int64_t", "int32_t *", u16, "int64_t",
                                          "int64_t *", "void *", "size_t", "void *"]
    assert _declaration("delta_diff_many") == [
        "int32_t", "const uint16_t * const *", "const uint16_t * const *", "const int64_t *",
        "int32_t *", u16, "int64_t", "int64_t *", "int64_t *", "void *", "size_t", "void *"]
    assert _declaration("delta_apply") == [u16, "int64_t", "const int32_t *", u16c, "int64_t",
                                           "void *"]
    assert _declaration("xor_mask") == [u16c, u16c, u16, "int64_t", "void *"]
    assert _declaration("xor_apply") == [u16, u16c, "int64_t", "void *"]
    assert _declaration("delta_last_error") == ["void"]


def test_noalloc_diff_argument_checks():
    """delta_diff_noalloc rejects what does not fit its static scratch, and bad
    arguments, before anything reaches the GPU."""
    lib = _abi.load()
    top = lib.delta_diff_noalloc_max_elems()
    assert top == 1 << 28
    # the fixed scratch regions for the largest accepted tensor leave a
    # staging arena of at least a quarter of the 48 MiB
    assert lib.delta_workspace_size_for(top, 1, 0) <= 36 << 20
    one = ctypes.c_void_p(16)
    assert lib.delta_diff_noalloc(one, one, top + 1, one, one, 5, one, None) == _abi.DELTA_E_RANGE
    assert "static scratch" in _err(lib)
    assert lib.delta_diff_noalloc(one, one, -1, one, one, 5, one, None) == _abi.DELTA_E_INVALID
    assert lib.delta_diff_noalloc(one, one, 10, one, one, -1, one, None) == _abi.DELTA_E_INVALID
    assert lib.delta_diff_noalloc(one, one, 10, one, one, 5, None, None) == _abi.DELTA_E_INVALID
    assert lib.delta_diff_noalloc(None, one, 10, one, one, 5, one, None) == _abi.DELTA_E_INVALID
    assert lib.delta_diff_noalloc(one, one, 10, None, one, 5, one, None) == _abi.DELTA_E_INVALID


def test_workspace_sizes_from_capacity():
    """The minimum workspace holds no arena; a capacity adds 4 bytes per kept
    entry (plus quad rounding per tile) up to the worst case."""
    lib = _abi.load()
    n, k = 6_738_415_616, 291
    worst = lib.delta_workspace_size(n, k)
    low = lib.delta_workspace_size_for(n, k, 0)
    mid = lib.delta_workspace_size_for(n, k, 80_000_000)
    assert low < mid < worst
    assert 4 * 80_000_000 <= mid - low <= 4 * 80_000_000 + 16 * (n // 32768 + k + 1) + 256
    assert lib.delta_workspace_size_for(n, k, n) == worst
    assert mid < 1 << 30  # the 7B-shaped list sized for about its headline delta's count
    assert lib.delta_workspace_size_for(-1, 1, 0) == 0
    assert lib.delta_workspace_size_for(1, 1, -1) == 0
    # capacities whose 4 bytes per entry pass the worst case (or int64) get it
    big = 1 << 62
    assert lib.delta_workspace_size_for(big, 1, big) == lib.delta_workspace_size(big, 1)
    top = (1 << 63) - 1
    assert lib.delta_workspace_size_for(top, 1, top) == lib.delta_workspace_size(top, 1) > 0
    # a diff accepts the minimum and rejects one byte less, before any launch
    one = ctypes.c_void_p(16)
    m1 = lib.delta_workspace_size_for(1 << 20, 1, 0)
    assert lib.delta_diff(one, one, 1 << 20, one, one, 5, one, ctypes.c_void_p(256), m1 - 1,
                          None) == _abi.DELTA_E_WORKSPACE
