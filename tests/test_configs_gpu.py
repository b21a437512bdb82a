"""GPU parity at the configurations' full sizes, in the launch configuration
the benchmark times (flat 256-byte-aligned arenas, DiffPlan / ApplyPlan).

The oracle compares every tensor of the 0.6B- and 7B-shaped lists and every
density-sweep case element for element (tolerance 0).  The 405B layer share
(64 GB per snapshot) is checked by properties that hold at any size -- the
per-parameter count equals torch's count of differing bit patterns, apply
turns the old snapshot into the new one, XOR round-trips -- plus the oracle on
sampled windows.
"""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


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


def torch_counts(olds, news):
    return [int((a.view(torch.int16) != b.view(torch.int16)).sum().item())
            for a, b in zip(olds, news)]


def check_whole_list(sbd, oracle_mod, olds, news, capacity):
    from sparse_bf16_delta_amd.plan import ApplyPlan, DiffPlan

    dp = DiffPlan(olds, news, capacity)
    dp.run()
    idx, val, nnz, offsets = dp.result()
    offs = offsets.cpu().numpy()
    nnz_h = nnz.cpu().numpy()
    assert np.array_equal(np.diff(offs), nnz_h)
    for p, (o, x) in enumerate(zip(olds, news)):
        ri, rv = oracle_mod.diff(bits(o), bits(x))
        assert nnz_h[p] == ri.size, p
        assert np.array_equal(idx[offs[p]:offs[p + 1]].cpu().numpy(), ri), p
        assert np.array_equal(bits(val[offs[p]:offs[p + 1]]), rv), p
    snaps = [o.clone() for o in olds]
    ApplyPlan(snaps).run(dp.idx, dp.val, dp.offsets, dp.capacity)
    for s, x in zip(snaps, news):
        assert torch.equal(s.view(torch.int16), x.view(torch.int16))
    return int(offs[-1])


def test_qwen3_0p6b_list_full(sbd, oracle_mod):
    cfg = workloads.CONFIGS["qwen3_0p6b"]
    old, new, olds, news, offs, numels = build_arenas(cfg, 3e-6, "fp32_master", "cuda")
    total = check_whole_list(sbd, oracle_mod, olds, news, cfg.total // 4)
    mask = sbd.xor_mask(old, new)
    snap = old.clone()
    sbd.xor_apply_(snap, mask)
    assert torch.equal(snap.view(torch.int16), new.view(torch.int16))
    assert int((mask != 0).sum().item()) == total
    print(f"qwen3-0.6B list: {total} of {cfg.total} changed ({total / cfg.total:.4%})")


def test_llama7b_headline_full(sbd, oracle_mod):
    """The benchmark's workload: bf16-resident step at lr 1e-6, every tensor
    compared with the oracle."""
    cfg = workloads.CONFIGS["llama7b"]
    old, new, olds, news, offs, numels = build_arenas(cfg, 1e-6, "bf16_resident", "cuda")
    total = check_whole_list(sbd, oracle_mod, olds, news, cfg.total // 8)
    print(f"llama-7B list lr 1e-6 bf16-resident: {total} changed ({total / cfg.total:.4%})")


@pytest.mark.parametrize("lr,mode", [(3e-6, "bf16_resident"), (1e-5, "bf16_resident"),
                                     (1e-6, "fp32_master"), (3e-6, "fp32_master"),
                                     (1e-5, "fp32_master")])
def test_llama7b_other_steps(sbd, oracle_mod, lr, mode):
    """Counts against torch for every tensor, apply identity for the list, and
    the oracle on three whole tensors."""
    from sparse_bf16_delta_amd.plan import ApplyPlan, DiffPlan

    cfg = workloads.CONFIGS["llama7b"]
    old, new, olds, news, offs, numels = build_arenas(cfg, lr, mode, "cuda")
    dp = DiffPlan(olds, news, cfg.total // 4)
    dp.run()
    idx, val, nnz, offsets = dp.result()
    assert nnz.cpu().tolist() == torch_counts(olds, news)
    off_h = offsets.cpu().numpy()
    for p in (0, 150, len(olds) - 1):
        ri, rv = oracle_mod.diff(bits(olds[p]), bits(news[p]))
        assert np.array_equal(idx[off_h[p]:off_h[p + 1]].cpu().numpy(), ri)
        assert np.array_equal(bits(val[off_h[p]:off_h[p + 1]]), rv)
    snap = old.clone()
    snaps = [snap[o:o + n] for o, n in zip(offs, numels)]
    ApplyPlan(snaps).run(dp.idx, dp.val, dp.offsets, dp.capacity)
    assert torch.equal(snap.view(torch.int16), new.view(torch.int16))
    total = int(off_h[-1])
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


def test_llama405b_share_sparse_path(sbd, oracle_mod, llama405b_share):
    """Layer by layer (7 tensors per diff_many): counts equal torch's, apply
    into a copy of the layer gives the new layer, and oracle windows agree."""
    from sparse_bf16_delta_amd.plan import ApplyPlan, DiffPlan

    cfg, old, new, olds, news = llama405b_share
    rng = np.random.default_rng(5)
    total = 0
    for layer in range(10):
        lo, ln = olds[7 * layer:7 * layer + 7], news[7 * layer:7 * layer + 7]
        n_layer = sum(t.numel() for t in lo)
        dp = DiffPlan(lo, ln, n_layer // 8)
        dp.run()
        idx, val, nnz, offsets = dp.result()
        assert nnz.cpu().tolist() == torch_counts(lo, ln)
        off_h = offsets.cpu().numpy()
        # oracle on a seeded window of one tensor of the layer
        p = int(rng.integers(0, 7))
        w0 = int(rng.integers(0, lo[p].numel() - (1 << 22)))
        w1 = w0 + (1 << 22)
        seg = idx[off_h[p]:off_h[p + 1]]
        a = int(torch.searchsorted(seg, torch.tensor([w0], dtype=torch.int32, device="cuda")).item())
        b = int(torch.searchsorted(seg, torch.tensor([w1], dtype=torch.int32, device="cuda")).item())
        ri, rv = oracle_mod.diff(bits(lo[p][w0:w1]), bits(ln[p][w0:w1]))
        assert np.array_equal(seg[a:b].cpu().numpy() - w0, ri)
        assert np.array_equal(bits(val[off_h[p] + a:off_h[p] + b]), rv)
        snaps = [t.clone() for t in lo]
        ApplyPlan(snaps).run(dp.idx, dp.val, dp.offsets, dp.capacity)
        for s, x in zip(snaps, ln):
            assert torch.equal(s.view(torch.int16), x.view(torch.int16))
        del snaps, dp
        total += int(off_h[-1])
    print(f"405B share: {total} of {cfg.total} changed ({total / cfg.total:.4%})")


def test_llama405b_share_xor_path(sbd, llama405b_share):
    """XOR mode in place over each layer: old ^ mask == new, and again restores."""
    cfg, old, new, olds, news = llama405b_share
    for layer in range(10):
        lo, ln = olds[7 * layer:7 * layer + 7], news[7 * layer:7 * layer + 7]
        for a, b in zip(lo, ln):
            mask = sbd.xor_mask(a, b)
            assert int((mask != 0).sum().item()) == int(
                (a.view(torch.int16) != b.view(torch.int16)).sum().item())
            sbd.xor_apply_(a, mask)
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
            sbd.xor_apply_(a, mask)
            del mask


def test_largest_tensor_int32_index_range(sbd, oracle_mod):
    """One tensor of 2^31 - 1 elements, the most the int32 index contract
    allows, about 2 % changed (the last and first elements among them): the
    count equals torch's count of differing bit patterns, the indices ascend
    strictly and the values are new's, apply (sparse workgroups rewriting
    whole segments) turns old into new, XOR round-trips, and the oracle
    agrees exactly on the first and last million elements."""
    n = (1 << 31) - 1
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    old = torch.randint(-(1 << 15), 1 << 15, (n,), dtype=torch.int16, device="cuda", generator=g)
    pick = torch.randint(0, 1000, (n,), dtype=torch.int16, device="cuda", generator=g) < 20
    pick[0] = True
    pick[n - 1] = True
    new = torch.where(pick, old ^ 0x1, old)
    want_count = int(pick.sum().item())
    del pick
    idx, val = sbd.diff(old.view(torch.bfloat16), new.view(torch.bfloat16))
    assert idx.numel() == want_count
    assert int(idx[0]) == 0 and int(idx[-1]) == n - 1
    assert bool((idx[1:] > idx[:-1]).all())
    assert torch.equal(val.view(torch.int16), new[idx.long()])
    w = 1 << 20
    for a in (0, n - w):
        lo = int(torch.searchsorted(idx, torch.tensor([a], dtype=torch.int32, device="cuda")))
        hi = int(torch.searchsorted(idx, torch.tensor([a + w], dtype=torch.int32, device="cuda")))
        ri, rv = oracle_mod.diff(bits(old[a:a + w]), bits(new[a:a + w]))
        assert np.array_equal(idx[lo:hi].cpu().numpy() - a, ri)
        assert np.array_equal(bits(val[lo:hi]), rv)
    snap = old.clone()
    assert idx.numel() >= (1 << 25)  # large enough for the segment rewrite
    sbd.apply_(snap.view(torch.bfloat16), idx, val, check_indices=True)
    assert torch.equal(snap, new)
    del idx, val
    mask = sbd.xor_mask(old.view(torch.bfloat16), new.view(torch.bfloat16))
    assert int((mask.view(torch.int16) != 0).sum().item()) == want_count
    sbd.xor_apply_(snap.view(torch.bfloat16), mask)
    assert torch.equal(snap, old)
