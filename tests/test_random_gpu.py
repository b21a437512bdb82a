"""Seeded random parameter lists, against the oracle, bit for bit.

Each seed draws a list packed back to back at odd element offsets in one
buffer (sizes from empty to several 32768-element tiles, many next to tile
and segment boundaries), a change density per parameter from none to all,
sometimes in contiguous runs, and a capacity that may cut the delta.  The
diff must give the oracle's true counts and offsets and, up to the cut, its
indices and values; the full delta applied to a copy of `old` must give
`new`; the XOR mask and its apply must match as well.  All inputs and
expected values come from numpy and the oracle; the seeds are fixed.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

TILE = 32768
SIZE_MENU = [0, 1, 2, 7, 8, 9, 31, 32, 33, 63, 64, 65, 1000, 2047, 2048, 2049, 4095, 4096,
             TILE - 1, TILE, TILE + 1, 2 * TILE - 5, 3 * TILE + 17]
FRAC_MENU = [0.0, 1e-4, 0.003, 0.01, 0.03, 0.08, 0.124, 0.126, 0.3, 0.7, 1.0]


@pytest.fixture(scope="module")
def sbd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_bf16_delta_amd as m

    m.load()
    return m


def np_bits(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)


def draw_case(seed):
    rng = np.random.default_rng(90_000 + seed)
    k = int(rng.integers(1, 24))
    sizes = [int(rng.choice(SIZE_MENU)) if rng.random() < 0.7 else int(rng.integers(0, 4 * TILE))
             for _ in range(k)]
    olds, news = [], []
    for n in sizes:
        old = rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
        new = old.copy()
        frac = float(rng.choice(FRAC_MENU))
        c = int(round(frac * n))
        if c:
            if rng.random() < 0.3:  # contiguous runs of changes
                run = int(rng.integers(1, 300))
                starts = rng.choice(max(n - run, 0) + 1, size=max(1, c // run), replace=True)
                pos = np.unique(np.concatenate([np.arange(s, min(s + run, n)) for s in starts]))
            else:
                pos = rng.choice(n, size=c, replace=False)
            new[pos] = (old[pos].astype(np.uint32)
                        + rng.integers(1, 1 << 16, size=pos.size, dtype=np.uint32)).astype(np.uint16)
        olds.append(old)
        news.append(new)
    gaps = [int(g) for g in rng.integers(0, 9, size=k)]  # odd element offsets between parameters
    return rng, sizes, gaps, olds, news


def pack(arrays, gaps, lead):
    """One device buffer holding the arrays back to back after `lead` elements,
    each followed by its gap; returns the buffer and views of the arrays."""
    total = lead + sum(a.size + g for a, g in zip(arrays, gaps))
    host = np.zeros(total, dtype=np.uint16)
    pos, spans = lead, []
    for a, g in zip(arrays, gaps):
        host[pos:pos + a.size] = a
        spans.append((pos, a.size))
        pos += a.size + g
    buf = torch.from_numpy(host.view(np.int16).copy()).cuda().view(torch.bfloat16)
    return buf, [buf[p:p + n] for p, n in spans], host


@pytest.mark.parametrize("seed", range(40))
def test_random_lists_match_oracle(sbd, oracle_mod, seed):
    from sparse_bf16_delta_amd.plan import DiffPlan

    rng, sizes, gaps, olds, news = draw_case(seed)
    ri, rv, rn, ro = oracle_mod.diff_many(olds, news)
    total = int(ro[-1])
    lead = int(rng.integers(0, 8))
    _, g_old, _ = pack(olds, gaps, lead)
    _, g_new, _ = pack(news, gaps, int(rng.integers(0, 8)))

    # the diff at a capacity that may cut the delta
    cap = total if rng.random() < 0.5 else int(rng.integers(0, total + 2))
    plan = DiffPlan(g_old, g_new, cap)
    plan.run()
    assert plan.changed() == total
    assert np.array_equal(plan.offsets.cpu().numpy(), ro)
    assert np.array_equal(plan.nnz.cpu().numpy(), rn)
    m = min(cap, total)
    assert np.array_equal(plan.idx[:m].cpu().numpy(), ri[:m])
    assert np.array_equal(np_bits(plan.val[:m]), rv[:m])

    # the full delta applied into a packed copy of old gives new; the gaps and
    # the lead stay untouched
    gi, gv, gn, go = sbd.diff_many(g_old, g_new)
    buf, snaps, host_old = pack(olds, gaps, lead)
    sbd.apply_many_(snaps, gi, gv, go, check_indices=True)
    want = host_old.copy()
    pos = lead
    for x, g in zip(news, gaps):
        want[pos:pos + x.size] = x
        pos += x.size + g
    assert np.array_equal(np_bits(buf), want)

    # XOR mode on every parameter
    for o, x, go_, gn_ in zip(olds, news, g_old, g_new):
        mask = sbd.xor_mask(go_, gn_)
        assert np.array_equal(np_bits(mask), oracle_mod.xor_mask(o, x))
        snap = go_.clone()
        sbd.xor_apply_(snap, mask)
        assert np.array_equal(np_bits(snap), x)


SMALL_MENU = [0, 0, 0, 1, 2, 31, 33, 64, 1000, 4096, 33_000, 70_000]


@pytest.mark.parametrize("k,seed", [(300, 0), (4100, 1), (9000, 2)])
def test_many_small_parameters_match_oracle(sbd, oracle_mod, k, seed):
    """Lists of hundreds to thousands of mostly tiny (often empty) tensors:
    the parameter searches take two and three 64-way steps, apply chunks
    straddle many parameters, and the placing walk crosses many small tiles.
    Diff, apply and both wire encodings match the oracle bit for bit."""
    from sparse_bf16_delta_amd.plan import DiffPlan

    rng = np.random.default_rng(70_000 + seed)
    sizes = [int(rng.choice(SMALL_MENU)) for _ in range(k)]
    olds, news = [], []
    for n in sizes:
        old = rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
        new = old.copy()
        c = int(round(float(rng.choice(FRAC_MENU)) * n))
        if c:
            pos = rng.choice(n, size=c, replace=False)
            new[pos] = (old[pos].astype(np.uint32)
                        + rng.integers(1, 1 << 16, size=c, dtype=np.uint32)).astype(np.uint16)
        olds.append(old)
        news.append(new)
    gaps = [int(g) for g in rng.integers(0, 3, size=k)]
    ri, rv, rn, ro = oracle_mod.diff_many(olds, news)
    _, g_old, host_old = pack(olds, gaps, 1)
    _, g_new, _ = pack(news, gaps, 3)

    plan = DiffPlan(g_old, g_new, int(ro[-1]))
    plan.run()
    assert plan.changed() == int(ro[-1])
    assert np.array_equal(plan.offsets.cpu().numpy(), ro)
    assert np.array_equal(plan.nnz.cpu().numpy(), rn)
    assert np.array_equal(plan.idx[:ro[-1]].cpu().numpy(), ri)
    assert np.array_equal(np_bits(plan.val[:ro[-1]]), rv)

    buf, snaps, host_old = pack(olds, gaps, 1)
    sbd.apply_many_(snaps, plan.idx[:ro[-1]], plan.val[:ro[-1]], plan.offsets, check_indices=True)
    want = host_old.copy()
    pos = 1
    for x, g in zip(news, gaps):
        want[pos:pos + x.size] = x
        pos += x.size + g
    assert np.array_equal(np_bits(buf), want)

    gi = plan.idx[:ro[-1]]
    want_pos, want_po = oracle_mod.wire_encode(ri, ro, sizes)
    wpos, wpo = sbd.wire_encode(gi, plan.offsets, sizes)
    assert np.array_equal(wpos.cpu().numpy(), want_pos)
    assert np.array_equal(wpo.cpu().numpy(), want_po)
    assert np.array_equal(sbd.wire_decode(wpos, wpo, plan.offsets, sizes).cpu().numpy(), ri)
    want_blk = oracle_mod.wire_encode_blocked(ri, ro, sizes)
    blk = sbd.wire_encode_blocked(gi, plan.offsets, sizes)
    assert np.array_equal(blk.cpu().numpy(), want_blk)
    assert np.array_equal(sbd.wire_decode_blocked(blk, plan.offsets, sizes).cpu().numpy(), ri)
    print(f"k={k}: {sum(sizes)} elements, {int(ro[-1])} changed", flush=True)
