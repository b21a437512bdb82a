"""delta_diff_noalloc -- the diff that allocates nothing -- through the C ABI.

Its output is compared with delta_diff's (the entry point with a caller
workspace) bit for bit -- count, indices, values -- and nothing is written
past the count.  Two calls in a row, the second on a smaller tensor, so the
second runs on a static scratch that still holds the first call's contents.
"""
import ctypes

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


def _delta(lib, fn, old, new, cap, ws=None):
    dev = old.device
    idx = torch.full((cap,), -7, dtype=torch.int32, device=dev)
    val = torch.full((cap,), -7, dtype=torch.int16, device=dev)
    nnz = torch.full((1,), -1, dtype=torch.int64, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    p = ctypes.c_void_p
    if ws is None:
        rc = fn(p(old.data_ptr()), p(new.data_ptr()), old.numel(), p(idx.data_ptr()),
                p(val.data_ptr()), cap, p(nnz.data_ptr()), st)
    else:
        rc = fn(p(old.data_ptr()), p(new.data_ptr()), old.numel(), p(idx.data_ptr()),
                p(val.data_ptr()), cap, p(nnz.data_ptr()), p(ws.data_ptr()), ws.numel(), st)
    assert rc == 0, lib.delta_last_error()
    torch.cuda.synchronize()
    return int(nnz.item()), idx, val


def test_noalloc_diff_matches_delta_diff_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_bf16_delta_amd import _abi

    lib = _abi.load()
    dev = torch.device("cuda:0")
    top = int(lib.delta_diff_noalloc_max_elems())
    # the largest tensor it takes, then a smaller, ragged one
    for n, seed in ((top, 11), (3 * 32768 + 17, 12)):
        old, new = workloads.make_step_pair(n, *workloads.seeds(1, seed), 3e-6, "fp32_master",
                                            device=dev)
        cap = n // 8 + 4096
        ws = torch.empty(lib.delta_workspace_size(n, 1), dtype=torch.uint8, device=dev)
        k_ref, i_ref, v_ref = _delta(lib, lib.delta_diff, old, new, cap, ws)
        k, i, v = _delta(lib, lib.delta_diff_noalloc, old, new, cap)
        assert 0 < k_ref <= cap
        assert k == k_ref
        assert torch.equal(i[:k], i_ref[:k]) and torch.equal(v[:k], v_ref[:k])
        assert bool((i[k:] == -7).all()) and bool((v[k:] == -7).all())
        print(f"n={n}: {k} changed, identical to delta_diff", flush=True)


def test_noalloc_diff_on_a_side_stream():
    """On a stream of its own (a non-null handle, checked to belong to the
    current device) the result is the same as delta_diff's on that stream."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_bf16_delta_amd import _abi

    lib = _abi.load()
    dev = torch.device("cuda:0")
    n = 5 * 32768 + 3
    old, new = workloads.make_step_pair(n, *workloads.seeds(1, 13), 3e-6, "fp32_master",
                                        device=dev)
    cap = n // 4
    ws = torch.empty(lib.delta_workspace_size(n, 1), dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        assert torch.cuda.current_stream(dev).cuda_stream != 0
        k_ref, i_ref, v_ref = _delta(lib, lib.delta_diff, old, new, cap, ws)
        k, i, v = _delta(lib, lib.delta_diff_noalloc, old, new, cap)
    assert 0 < k_ref <= cap and k == k_ref
    assert torch.equal(i[:k], i_ref[:k]) and torch.equal(v[:k], v_ref[:k])
