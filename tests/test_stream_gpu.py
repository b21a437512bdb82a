"""GPU parity of the streamed receiver: a delta (or XOR mask) in host memory,
copied and applied chunk by chunk, must give exactly what the oracle's apply
gives -- every chunking, pinned or pageable host buffers."""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

TILE = 32768


@pytest.fixture(scope="module")
def sbd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_bf16_delta_amd as m

    m.load()
    return m


def np_bits(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)


def rand_pair(seed, n, frac):
    rng = np.random.default_rng(seed)
    old = rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
    new = old.copy()
    k = int(round(frac * n))
    if k:
        pos = rng.choice(n, size=k, replace=False)
        off = rng.integers(1, 1 << 16, size=k, dtype=np.uint32).astype(np.uint16)
        new[pos] = (old[pos].astype(np.uint32) + off).astype(np.uint16)
    return old, new


SIZES = [128, 0, TILE, 1, TILE + 1, 1024, 0, 3 * TILE - 1, 128, 7, 65536, 33_000, 5 * TILE + 3]


@pytest.mark.parametrize("bounds", [
    [0, len(SIZES)],                       # one chunk
    list(range(len(SIZES) + 1)),           # one parameter per chunk
    [0, 3, 3, 7, 7, 7, len(SIZES)],        # empty chunks in between
    [0, 1, 2, 5, 11, len(SIZES)],
])
@pytest.mark.parametrize("pinned", [True, False])
@pytest.mark.parametrize("frac", [0.01, 0.2, 0.7])
def test_apply_streamed_matches_oracle(sbd, oracle_mod, bounds, pinned, frac):
    olds, news = zip(*[rand_pair(100 * i + int(frac * 50), s, frac) for i, s in enumerate(SIZES)])
    ri, rv, rn, ro = oracle_mod.diff_many(olds, news)
    want = []
    for o, x in zip(olds, news):
        w = o.copy()
        oracle_mod.apply_(w, *oracle_mod.diff(o, x))
        want.append(w)
    idx = torch.from_numpy(ri.copy())
    val = torch.from_numpy(rv.view(np.int16).copy()).view(torch.bfloat16)
    off = torch.from_numpy(ro.copy())
    if pinned:
        idx, val, off = idx.pin_memory(), val.pin_memory(), off.pin_memory()
    snaps = [torch.from_numpy(o.view(np.int16).copy()).cuda().view(torch.bfloat16) for o in olds]
    sbd.apply_streamed_(snaps, idx, val, off, bounds)
    for s, w in zip(snaps, want):
        assert np.array_equal(np_bits(s), w)


def test_apply_streamed_tile_kinds_from_device_diff(sbd, oracle_mod):
    """The sender's diff_many output, moved to pinned host memory, streamed
    back into a copy of the old snapshots gives the new ones."""
    cfg = workloads.CONFIGS["qwen3_0p6b"]
    params = list(range(0, len(cfg.params), 7))[:40]
    numels = [cfg.numels[t] for t in params]
    offs, n_alloc = workloads.flat_layout(numels)
    old = torch.zeros(n_alloc, dtype=torch.bfloat16, device="cuda")
    new = torch.zeros(n_alloc, dtype=torch.bfloat16, device="cuda")
    for t, o, n in zip(params, offs, numels):
        workloads.fill_step_pair_(old[o:o + n], new[o:o + n], *workloads.seeds(cfg.seed_family, t),
                                  3e-6, "fp32_master")
    olds = [old[o:o + n] for o, n in zip(offs, numels)]
    news = [new[o:o + n] for o, n in zip(offs, numels)]
    gi, gv, gn, go = sbd.diff_many(olds, news)
    snap = old.clone()
    snaps = [snap[o:o + n] for o, n in zip(offs, numels)]
    bounds = list(range(0, len(params), 4)) + [len(params)]
    sbd.apply_streamed_(snaps, gi.cpu().pin_memory(), gv.cpu().pin_memory(),
                        go.cpu().pin_memory(), bounds)
    assert torch.equal(snap.view(torch.int16), new.view(torch.int16))


@pytest.mark.parametrize("n,chunk", [(0, 64), (1, 64), (1000, 64), (100_003, 4096),
                                     (3 * TILE + 5, TILE), (1 << 20, 1 << 20), (1 << 20, 999)])
@pytest.mark.parametrize("pinned", [True, False])
def test_xor_apply_streamed_matches_oracle(sbd, oracle_mod, n, chunk, pinned):
    old, new = rand_pair(n + chunk, n, 0.05)
    mask = oracle_mod.xor_mask(old, new)
    want = old.copy()
    oracle_mod.xor_apply_(want, mask)
    h = torch.from_numpy(mask.view(np.int16).copy()).view(torch.bfloat16)
    if pinned and n:
        h = h.pin_memory()
    snap = torch.from_numpy(old.view(np.int16).copy()).cuda().view(torch.bfloat16)
    sbd.xor_apply_streamed_(snap, h, chunk_elems=chunk)
    assert np.array_equal(np_bits(snap), want)


def test_streamed_apply_plan_reused_over_steps(sbd, oracle_mod):
    """A plan built once applies successive steps' host deltas (forward, then
    the reverse delta back to the start), and rejects a chunk larger than it
    was sized for."""
    from sparse_bf16_delta_amd.plan import StreamedApplyPlan

    olds, news = zip(*[rand_pair(7 * i + 1, s, 0.05) for i, s in enumerate(SIZES)])
    fwd = oracle_mod.diff_many(olds, news)
    rev = oracle_mod.diff_many(news, olds)
    snaps = [torch.from_numpy(o.view(np.int16).copy()).cuda().view(torch.bfloat16) for o in olds]
    bounds = [0, 4, 9, len(SIZES)]

    def host(d):
        i, v, n, o = d
        return (torch.from_numpy(i.copy()).pin_memory(),
                torch.from_numpy(v.view(np.int16).copy()).view(torch.bfloat16).pin_memory(),
                torch.from_numpy(o.copy()).pin_memory())

    hf, hr = host(fwd), host(rev)
    biggest = max(int(d[3][hi] - d[3][lo]) for d in (fwd, rev) for lo, hi in zip(bounds, bounds[1:]))
    plan = StreamedApplyPlan(snaps, bounds, biggest)
    for step in range(3):
        plan.run(*hf)
        assert all(np.array_equal(np_bits(s), x) for s, x in zip(snaps, news))
        plan.run(*hr)
        assert all(np.array_equal(np_bits(s), o) for s, o in zip(snaps, olds))
    small = StreamedApplyPlan(snaps, bounds, 1)
    with pytest.raises(sbd.DeltaError, match="more than"):
        small.run(*hf)


# ---- the host-direct receiver: the apply kernel reads the pinned host delta

@pytest.mark.parametrize("frac", [0.0, 0.01, 0.2, 0.7])
def test_apply_many_host_matches_oracle(sbd, oracle_mod, frac):
    """delta_apply_many_host reads idx and val straight from pinned host
    memory; the snapshots end exactly as the oracle's apply leaves them."""
    olds, news = [], []
    for i, n in enumerate(SIZES):
        o, x = rand_pair(400 + i + int(frac * 1000), n, frac)
        olds.append(o)
        news.append(x)
    ri, rv, rn, ro = oracle_mod.diff_many(olds, news)
    snaps = [torch.from_numpy(o.view(np.int16)).cuda() for o in olds]
    # views into larger pinned buffers, starting past their first element
    h_idx = torch.zeros(ri.size + 5, dtype=torch.int32).pin_memory()[3:3 + ri.size]
    h_val = torch.zeros(rv.size + 5, dtype=torch.int16).pin_memory()[1:1 + rv.size]
    h_idx.copy_(torch.from_numpy(ri))
    h_val.copy_(torch.from_numpy(rv.view(np.int16)))
    sbd.apply_many_host_(snaps, h_idx, h_val.view(torch.bfloat16), torch.from_numpy(ro),
                         check_indices=True)
    for s, x in zip(snaps, news):
        assert np.array_equal(np_bits(s), x)


def test_apply_many_host_from_device_diff_and_back(sbd, oracle_mod):
    """A sender's diff_many output moved to pinned host memory, applied by the
    host-direct path, then the reverse delta likewise: back to old."""
    olds, news = [], []
    for i, n in enumerate(SIZES):
        o, x = rand_pair(500 + i, n, 0.05)
        olds.append(o)
        news.append(x)
    g_o = [torch.from_numpy(o.view(np.int16)).cuda() for o in olds]
    g_n = [torch.from_numpy(x.view(np.int16)).cuda() for x in news]
    snaps = [t.clone() for t in g_o]
    for src, dst, want in ((g_o, g_n, news), (g_n, g_o, olds)):
        gi, gv, gn, go = sbd.diff_many(src, dst)
        sbd.apply_many_host_(snaps, gi.cpu().pin_memory(), gv.cpu().pin_memory(), go.cpu())
        for s, w in zip(snaps, want):
            assert np.array_equal(np_bits(s), w)


def test_apply_many_host_rejects_unpinned_and_bad_offsets(sbd):
    """Pageable host buffers and malformed offsets are refused before any
    launch; the snapshot is untouched."""
    from sparse_bf16_delta_amd import _abi
    from sparse_bf16_delta_amd.ops import _ptr, _stream
    import ctypes

    snap = torch.arange(1000, dtype=torch.int16, device="cuda")
    before = snap.clone()
    idx = torch.tensor([1, 5, 9], dtype=torch.int32)
    val = torch.tensor([7, 7, 7], dtype=torch.int16)
    off = torch.tensor([0, 3], dtype=torch.int64)
    with pytest.raises(ValueError, match="pinned"):
        sbd.apply_many_host_([snap], idx, val.view(torch.bfloat16), off)
    lib = _abi.load()
    ws = torch.empty(lib.delta_workspace_size(0, 1), dtype=torch.uint8, device="cuda")
    sp = (ctypes.c_void_p * 1)(snap.data_ptr())
    nums = (ctypes.c_int64 * 1)(1000)
    # the ABI itself refuses pageable memory (it is not mapped for the GPU)
    st = lib.delta_apply_many_host(1, sp, nums, _ptr(idx), _ptr(val), _ptr(off), 3, None,
                                   _ptr(ws), ws.numel(), _stream(snap.device))
    assert st == _abi.DELTA_E_INVALID and b"pinned" in lib.delta_last_error()
    p_idx, p_val = idx.pin_memory(), val.pin_memory()
    # the arrays must hold every entry the offsets name
    big = torch.tensor([0, 1 << 30], dtype=torch.int64)
    st = lib.delta_apply_many_host(1, sp, nums, _ptr(p_idx), _ptr(p_val), _ptr(big), 1 << 30,
                                   None, _ptr(ws), ws.numel(), _stream(snap.device))
    assert st == _abi.DELTA_E_INVALID
    bad = torch.tensor([1, 3], dtype=torch.int64)
    st = lib.delta_apply_many_host(1, sp, nums, _ptr(p_idx), _ptr(p_val), _ptr(bad), 3, None,
                                   _ptr(ws), ws.numel(), _stream(snap.device))
    assert st == _abi.DELTA_E_INVALID and b"offsets[0]" in lib.delta_last_error()
    # the streamed receiver refuses a val shorter than idx before any copy
    with pytest.raises(ValueError, match="equal length"):
        sbd.apply_streamed_([snap], p_idx, p_val[:2].view(torch.bfloat16), off, [0, 1])
    torch.cuda.synchronize()
    assert torch.equal(snap, before)
    assert torch.equal(snap, before)
    sbd.apply_many_host_([snap], p_idx, p_val.view(torch.bfloat16), off)
    assert [int(snap[i]) for i in (1, 5, 9)] == [7, 7, 7]
