"""GPU parity at the configurations' full sizes, in the launch configuration
the benchmark times (flat 256-byte-aligned arenas, DiffPlan / ApplyPlan).

Every tensor of every configuration is compared with the oracle element for
element (tolerance 0): the count, the order of the indices and the values of
its delta, and for the XOR mode its mask.  The oracle runs on host copies of
the very same bits, one tensor per task in a pool of threads (its C calls
release the interpreter lock), so the 64 GB-per-snapshot 405B share is
checked whole, layer by layer.  Apply is checked by its result (the snapshot
becomes `new`, bit for bit) with the delta's exact entry count and with a
capacity far above it, which launch different kernels.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

# oracle tasks at once; each holds a tensor's host copies (at most about
# 10 GB for the largest 405B tensor)
WORKERS = 8


@pytest.fixture(scope="module")
def sbd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_bf16_delta_amd as m

    m.load()
    return m


def bits(t):
    return workloads.bits_numpy(t)


def build_arenas(cfg, lr, mode, dev, params=None):
    params = params if params is not None else list(range(len(cfg.params)))
    numels = [cfg.numels[t] for t in params]
    offs, n_alloc = workloads.flat_layout(numels)
    old = torch.zeros(n_alloc, dtype=torch.bfloat16, device=dev)
    new = torch.zeros(n_alloc, dtype=torch.bfloat16, device=dev)
    for t, o, n in zip(params, offs, numels):
        workloads.fill_step_pair_(old[o:o + n], new[o:o + n], *workloads.seeds(cfg.seed_family, t),
                                  lr, mode)
    olds = [old[o:o + n] for o, n in zip(offs, numels)]
    news = [new[o:o + n] for o, n in zip(offs, numels)]
    return old, new, olds, news, offs, numels


def _pool_all(fn, items):
    """Run fn over items in the oracle thread pool; returns the items for
    which fn returned False (largest tensors first, so the pool ends even)."""
    with ThreadPoolExecutor(WORKERS) as ex:
        return [p for p, ok in ex.map(lambda p: (p, fn(p)), items) if not ok]


def compare_delta_with_oracle(oracle_mod, olds, news, idx, val, offsets):
    """Every parameter's slice of a diff_many result equals the oracle's diff
    of that parameter: same count, same indices in the same order, same
    values."""
    off = offsets.cpu().tolist()
    assert len(off) == len(olds) + 1 and off[0] == 0

    def one(p):
        ri, rv = oracle_mod.diff(bits(olds[p]), bits(news[p]))
        if off[p + 1] - off[p] != ri.size:
            return False
        gi = idx[off[p]:off[p + 1]].cpu().numpy()
        gv = bits(val[off[p]:off[p + 1]])
        return bool(np.array_equal(gi, ri) and np.array_equal(gv, rv))

    order = sorted(range(len(olds)), key=lambda p: -olds[p].numel())
    bad = _pool_all(one, order)
    assert not bad, f"parameters differing from the oracle: {bad[:10]}"
    return off[-1]


def compare_xor_with_oracle(sbd, oracle_mod, olds, news):
    """Every parameter's XOR mask equals the oracle's, and xor_apply of it
    turns a copy of old into new."""

    def one(p):
        mask = sbd.xor_mask(olds[p], news[p])
        want = oracle_mod.xor_mask(bits(olds[p]), bits(news[p]))
        ok = np.array_equal(bits(mask), want)
        snap = olds[p].clone()
        sbd.xor_apply_(snap, mask)
        ok = ok and torch.equal(snap.view(torch.int16), news[p].view(torch.int16))
        del mask, snap
        return ok

    order = sorted(range(len(olds)), key=lambda p: -olds[p].numel())
    bad = _pool_all(one, order)
    assert not bad, f"XOR masks differing from the oracle: {bad[:10]}"


def delta_properties_on_device(olds, news, idx, val, offsets):
    """Checks that hold for any correct delta, on the GPU: per parameter the
    indices ascend strictly inside the tensor, each names a changed element
    and carries new's bits there, and the count equals torch's count of
    changed elements (together: the delta is exactly {i : old[i] != new[i]})."""
    off = offsets.cpu().tolist()
    for p, (o, x) in enumerate(zip(olds, news)):
        i = idx[off[p]:off[p + 1]].long()
        v = val[off[p]:off[p + 1]].view(torch.int16)
        ov, nv = o.view(torch.int16), x.view(torch.int16)
        assert off[p + 1] - off[p] == int((ov != nv).sum().item()), p
        if i.numel():
            assert int(i[0]) >= 0 and int(i[-1]) < o.numel(), p
            assert bool((i[1:] > i[:-1]).all()), p
            assert torch.equal(v, nv[i]), p
            assert bool((ov[i] != nv[i]).all()), p


def apply_both_ways(olds, news, dp, total):
    """ApplyPlan with the exact count and with the plan's capacity: each turns
    a copy of old into new."""
    from sparse_bf16_delta_amd.plan import ApplyPlan

    for max_nnz in (total, dp.capacity):
        snaps = [o.clone() for o in olds]
        ApplyPlan(snaps).run(dp.idx, dp.val, dp.offsets, max_nnz)
        for p, (s, x) in enumerate(zip(snaps, news)):
            assert torch.equal(s.view(torch.int16), x.view(torch.int16)), (max_nnz, p)
        del snaps


def check_whole_list(sbd, oracle_mod, olds, news, capacity):
    from sparse_bf16_delta_amd.plan import DiffPlan

    dp = DiffPlan(olds, news, capacity)
    dp.run()
    idx, val, nnz, offsets = dp.result()
    assert np.array_equal(np.diff(offsets.cpu().numpy()), nnz.cpu().numpy())
    total = compare_delta_with_oracle(oracle_mod, olds, news, idx, val, offsets)
    apply_both_ways(olds, news, dp, total)
    return total


def test_qwen3_0p6b_list_full(sbd, oracle_mod):
    cfg = workloads.CONFIGS["qwen3_0p6b"]
    old, new, olds, news, offs, numels = build_arenas(cfg, 3e-6, "fp32_master", "cuda")
    total = check_whole_list(sbd, oracle_mod, olds, news, cfg.total // 4)
    compare_xor_with_oracle(sbd, oracle_mod, olds, news)
    mask = sbd.xor_mask(old, new)  # the whole arena at once, as the bench runs it
    snap = old.clone()
    sbd.xor_apply_(snap, mask)
    assert torch.equal(snap.view(torch.int16), new.view(torch.int16))
    assert int((mask != 0).sum().item()) == total
    print(f"qwen3-0.6B list: {total} of {cfg.total} changed ({total / cfg.total:.4%})")


@pytest.mark.parametrize("lr,mode", [(1e-6, "bf16_resident"), (3e-6, "bf16_resident"),
                                     (1e-5, "bf16_resident"), (1e-6, "fp32_master"),
                                     (3e-6, "fp32_master"), (1e-5, "fp32_master")])
def test_llama7b_step_full(sbd, oracle_mod, lr, mode):
    """Every tensor of the 7B-shaped list at every step the configuration
    names (lr 1e-6 bf16-resident is the benchmark's workload), against the
    oracle, with apply (exact count and capacity) and the XOR mode."""
    cfg = workloads.CONFIGS["llama7b"]
    old, new, olds, news, offs, numels = build_arenas(cfg, lr, mode, "cuda")
    total = check_whole_list(sbd, oracle_mod, olds, news, cfg.total // 4)
    compare_xor_with_oracle(sbd, oracle_mod, olds, news)
    print(f"llama-7B list lr {lr:g} {mode}: {total} changed ({total / cfg.total:.4%})")


@pytest.mark.parametrize("pattern", ["uniform", "clustered"])
@pytest.mark.parametrize("di,frac", list(enumerate(workloads.DENSITIES)))
def test_density_sweep_flat_2p28(sbd, oracle_mod, pattern, di, frac):
    n = 1 << 28
    old, new, k = workloads.density_case(n, frac, pattern, di, device="cuda")
    gi, gv = sbd.diff(old, new, capacity=k + 1024)
    assert gi.numel() == k
    ri, rv = oracle_mod.diff(bits(old), bits(new))
    assert np.array_equal(gi.cpu().numpy(), ri)
    assert np.array_equal(bits(gv), rv)
    snap = old.clone()
    sbd.apply_(snap, gi, gv)
    assert torch.equal(snap.view(torch.int16), new.view(torch.int16))
    mask = sbd.xor_mask(old, new)
    assert np.array_equal(bits(mask), oracle_mod.xor_mask(bits(old), bits(new)))
    sbd.xor_apply_(snap, mask)
    assert torch.equal(snap.view(torch.int16), old.view(torch.int16))


@pytest.fixture(scope="module")
def llama405b_share():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = workloads.CONFIGS["llama405b_share"]
    old, new, olds, news, offs, numels = build_arenas(cfg, 3e-6, "fp32_master", "cuda")
    torch.cuda.synchronize()
    yield cfg, old, new, olds, news
    del old, new, olds, news
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layer", range(10))
def test_llama405b_share_sparse_path(sbd, oracle_mod, llama405b_share, layer):
    """One layer of the 405B share (7 tensors per diff_many, as the bench
    streams it): every tensor's delta equals the oracle's, the on-device
    properties hold, and apply (exact count and capacity) gives the new
    layer."""
    from sparse_bf16_delta_amd.plan import DiffPlan

    cfg, old, new, olds, news = llama405b_share
    lo, ln = olds[7 * layer:7 * layer + 7], news[7 * layer:7 * layer + 7]
    n_layer = sum(t.numel() for t in lo)
    dp = DiffPlan(lo, ln, n_layer // 8)
    dp.run()
    idx, val, nnz, offsets = dp.result()
    total = compare_delta_with_oracle(oracle_mod, lo, ln, idx, val, offsets)
    delta_properties_on_device(lo, ln, idx, val, offsets)
    apply_both_ways(lo, ln, dp, total)
    print(f"405B share layer {layer}: {total} of {n_layer} changed ({total / n_layer:.4%})")


@pytest.mark.parametrize("layer", range(10))
def test_llama405b_share_xor_path(sbd, oracle_mod, llama405b_share, layer):
    """XOR mode over one layer: every tensor's mask equals the oracle's and
    xor_apply turns old into new; then in place on the resident tensors,
    twice (self-inverse), as the bench runs it."""
    cfg, old, new, olds, news = llama405b_share
    lo, ln = olds[7 * layer:7 * layer + 7], news[7 * layer:7 * layer + 7]
    compare_xor_with_oracle(sbd, oracle_mod, lo, ln)
    for a, b in zip(lo, ln):
        mask = sbd.xor_mask(a, b)
        sbd.xor_apply_(a, mask)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        sbd.xor_apply_(a, mask)
        del mask


def test_largest_tensor_int32_index_range(sbd, oracle_mod):
    """One tensor of 2^31 - 1 elements, the most the int32 index contract
    allows, about 2 % changed (the last and first elements among them): the
    delta equals the oracle's element for element, apply (sparse chunks
    rewriting whole segments) turns old into new, and the XOR mask equals
    the oracle's and round-trips."""
    n = (1 << 31) - 1
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    old = torch.randint(-(1 << 15), 1 << 15, (n,), dtype=torch.int16, device="cuda", generator=g)
    pick = torch.randint(0, 1000, (n,), dtype=torch.int16, device="cuda", generator=g) < 20
    pick[0] = True
    pick[n - 1] = True
    new = torch.where(pick, old ^ 0x1, old)
    del pick
    idx, val = sbd.diff(old.view(torch.bfloat16), new.view(torch.bfloat16))
    assert int(idx[0]) == 0 and int(idx[-1]) == n - 1
    ho, hn = bits(old), bits(new)
    ri, rv = oracle_mod.diff(ho, hn)
    assert np.array_equal(idx.cpu().numpy(), ri)
    assert np.array_equal(bits(val), rv)
    del ri, rv
    snap = old.clone()
    assert idx.numel() >= (1 << 25)  # large enough for the segment rewrite
    sbd.apply_(snap.view(torch.bfloat16), idx, val, check_indices=True)
    assert torch.equal(snap, new)
    del idx, val
    mask = sbd.xor_mask(old.view(torch.bfloat16), new.view(torch.bfloat16))
    assert np.array_equal(bits(mask), oracle_mod.xor_mask(ho, hn))
    sbd.xor_apply_(snap.view(torch.bfloat16), mask)
    assert torch.equal(snap, old)
