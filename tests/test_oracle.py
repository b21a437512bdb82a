"""Pins for the CPU oracle: each test checks it against something other than
itself -- values the pages print, closed forms from IEEE 754, invariants the
method guarantees, an independent library formulation, or brute force.

Sources are the pages' titles and sections:
  TRL  -- "Shipping a Trillion Parameters With a Hub Bucket: Delta Weight Sync in TRL"
  VERL -- verl PR #6974 review ("delta_sharded" checkpoint engine)
  XOR  -- humans& weight-sync summary (bitwise XOR mask)
"""
import numpy as np
import pytest
import torch

from conftest import read_golden
import workloads

# ----------------------------------------------------------------------------
# helpers that do not use the oracle
# ----------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns by widening to float32 (upper half)."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rand_bits(rng, n, changed_frac, special=False):
    old = rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
    new = old.copy()
    k = int(round(changed_frac * n))
    if k:
        pos = rng.choice(n, size=k, replace=False)
        # any different pattern: add a nonzero offset modulo 2^16
        off = rng.integers(1, 1 << 16, size=k, dtype=np.uint32).astype(np.uint16)
        new[pos] = (old[pos].astype(np.uint32) + off).astype(np.uint16)
    if special and n >= 8:
        # signed zeros, equal NaNs, NaN payload change, infinities
        old[:8] = [0x0000, 0x7FC0, 0x7FC0, 0x7F80, 0x8000, 0x0001, 0xFF80, 0x3F80]
        new[:8] = [0x8000, 0x7FC0, 0x7FC1, 0x7F80, 0x0000, 0x0001, 0x7F80, 0x3F80]
    return old, new


# ----------------------------------------------------------------------------
# golden fixtures printed on the pages
# ----------------------------------------------------------------------------


def test_golden_sync_log_sparsity(oracle_mod):
    """TRL section 4.2 log line: 1,234,567 of 200,000,000 changed -> 99.38 %."""
    g = read_golden("sync_log_sparsity.txt")
    s = oracle_mod.sparsity(int(g["changed"]), int(g["total"]))
    assert f"{100 * s:.2f}" == g["printed_percent"]
    assert f"{s:.4f}" == g["metadata_sparsity"]
    assert oracle_mod.sparsity(0, 10) == 1.0
    assert oracle_mod.sparsity(10, 10) == 0.0
    assert oracle_mod.sparsity(0, 0) == 0.0


def test_golden_wire_layout(oracle_mod):
    """TRL section 4.1 / VERL encode.py: int32 positions + bf16 values = 6 B each."""
    g = read_golden("wire_layout.txt")
    rng = np.random.default_rng(7)
    old, new = rand_bits(rng, 1000, 0.05)
    idx, val = oracle_mod.diff(old, new)
    assert idx.dtype == np.int32 and idx.itemsize == int(g["index_bytes"])
    assert val.dtype == np.uint16 and val.itemsize == int(g["value_bytes"])
    wire = idx.nbytes + val.size * val.itemsize
    assert wire == int(g["bytes_per_changed_element"]) * idx.size == 6 * 50


# ----------------------------------------------------------------------------
# diff: worked examples and invariants
# ----------------------------------------------------------------------------


def test_diff_worked_bit_patterns(oracle_mod):
    """Integer-view compare (VERL shard_delta_indices): bit patterns decide.

    +0 -> -0 is a change (a float compare would miss it); an unchanged NaN bit
    pattern is not a change (a float compare would always report it); a NaN
    payload change, -Inf -> +Inf and a subnormal change are changes."""
    old = np.array([0x0000, 0x7FC0, 0x7FC0, 0x3F80, 0xFF80, 0x0001, 0x3F80, 0x8000],
                   dtype=np.uint16)
    new = np.array([0x8000, 0x7FC0, 0x7FC1, 0x3F80, 0x7F80, 0x0002, 0x3F80, 0x8000],
                   dtype=np.uint16)
    idx, val = oracle_mod.diff(old, new)
    assert idx.tolist() == [0, 2, 4, 5]
    assert val.tolist() == [0x8000, 0x7FC1, 0x7F80, 0x0002]


@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 63, 64, 65, 511, 512, 513, 16383, 16385])
@pytest.mark.parametrize("frac", [0.0, 0.01, 0.5, 1.0])
def test_diff_invariants(oracle_mod, n, frac):
    """apply(old, diff(old,new)) == new; each index differs; strictly ascending;
    untouched positions unchanged -- together these fix the output uniquely."""
    rng = np.random.default_rng(1000 * n + int(frac * 100))
    old, new = rand_bits(rng, n, frac, special=True)
    idx, val = oracle_mod.diff(old, new)
    assert idx.dtype == np.int32 and val.dtype == np.uint16
    if idx.size:
        assert np.all(np.diff(idx.astype(np.int64)) > 0)
        assert idx[0] >= 0 and idx[-1] < n
        assert np.all(old[idx] != new[idx])
        assert np.array_equal(val, new[idx])
    snap = old.copy()
    oracle_mod.apply_(snap, idx, val)
    assert np.array_equal(snap, new)
    untouched = np.ones(n, dtype=bool)
    untouched[idx] = False
    assert np.array_equal(old[untouched], new[untouched])


def test_diff_matches_view_nonzero_formulation(oracle_mod):
    """The VERL formulation -- integer views, `!=`, `nonzero`, gather -- run
    through numpy gives the same (idx, val)."""
    rng = np.random.default_rng(11)
    for n, frac in [(100_000, 0.01), (70_001, 0.3), (4096, 1.0)]:
        old, new = rand_bits(rng, n, frac, special=True)
        ref_idx = np.flatnonzero(old.view(np.int16) != new.view(np.int16))
        idx, val = oracle_mod.diff(old, new)
        assert np.array_equal(idx, ref_idx.astype(np.int32))
        assert np.array_equal(val, new[ref_idx])


def test_diff_identical_inputs_empty(oracle_mod):
    """VERL test name: no change gives an empty delta."""
    rng = np.random.default_rng(3)
    x = rng.integers(0, 1 << 16, size=5000, dtype=np.uint32).astype(np.uint16)
    idx, val = oracle_mod.diff(x, x.copy())
    assert idx.size == 0 and val.size == 0


def test_diff_rejects_int32_overflow(oracle_mod):
    """VERL risks section: positions are int32; more than 2^31-1 elements must
    fail loudly rather than wrap.  The size check precedes any access."""
    lib = oracle_mod._load()
    a = np.zeros(1, dtype=np.uint16)
    i = np.zeros(1, dtype=np.int32)
    assert lib.oracle_diff(a.ctypes.data, a.ctypes.data, 1 << 31, i.ctypes.data,
                           a.ctypes.data) == -1
    assert lib.oracle_diff(a.ctypes.data, a.ctypes.data, -1, i.ctypes.data,
                           a.ctypes.data) == -1


# ----------------------------------------------------------------------------
# apply
# ----------------------------------------------------------------------------


def test_apply_precondition_violations_leave_snapshot(oracle_mod):
    snap = np.arange(10, dtype=np.uint16)
    before = snap.copy()
    for bad in ([3, 2], [1, 1], [0, 10], [-1, 4]):
        with pytest.raises(ValueError):
            oracle_mod.apply_(snap, np.array(bad, dtype=np.int32),
                              np.array([9, 9], dtype=np.uint16))
        assert np.array_equal(snap, before)
    oracle_mod.apply_(snap, np.array([], dtype=np.int32), np.array([], dtype=np.uint16))
    assert np.array_equal(snap, before)


def test_apply_replay_and_reverse(oracle_mod):
    """TRL section 4.1: a new replica loads an anchor and replays the deltas
    after it.  apply(apply(s0, d01), d12) == s2, and diff(new, old) undoes."""
    rng = np.random.default_rng(5)
    s0, s1 = rand_bits(rng, 50_000, 0.02)
    _, s2 = rand_bits(rng, 50_000, 0.02)
    s2 = np.where(rng.random(50_000) < 0.5, s1, s2).astype(np.uint16)
    d01, d12 = oracle_mod.diff(s0, s1), oracle_mod.diff(s1, s2)
    snap = s0.copy()
    oracle_mod.apply_(snap, *d01)
    oracle_mod.apply_(snap, *d12)
    assert np.array_equal(snap, s2)
    back = oracle_mod.diff(s2, s0)
    oracle_mod.apply_(snap, *back)
    assert np.array_equal(snap, s0)


# ----------------------------------------------------------------------------
# XOR mode
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("n", [0, 1, 9, 4097, 100_003])
def test_xor_roundtrip_and_cross_mode(oracle_mod, n):
    """XOR summary: new = old XOR mask exactly; applying twice restores;
    the mask is nonzero exactly where the sparse diff reports a change, and
    old[idx] XOR mask[idx] == val."""
    rng = np.random.default_rng(n + 17)
    old, new = rand_bits(rng, n, 0.03, special=True)
    mask = oracle_mod.xor_mask(old, new)
    # independent check with numpy's bitwise_xor
    assert np.array_equal(mask, np.bitwise_xor(old, new))
    snap = old.copy()
    oracle_mod.xor_apply_(snap, mask)
    assert np.array_equal(snap, new)
    oracle_mod.xor_apply_(snap, mask)
    assert np.array_equal(snap, old)
    idx, val = oracle_mod.diff(old, new)
    assert np.array_equal(np.flatnonzero(mask), idx.astype(np.int64))
    assert np.array_equal(np.bitwise_xor(old[idx], mask[idx]), val)


# ----------------------------------------------------------------------------
# diff_many
# ----------------------------------------------------------------------------


def test_diff_many_concatenates_in_order(oracle_mod):
    """VERL gather_v_batched_to_rank0 / DeltaParam: deltas of K parameters are
    concatenated in list order with a count vector; indices stay local."""
    rng = np.random.default_rng(9)
    sizes = [128, 0, 1024, 1, 33_000, 128, 7]
    olds, news = [], []
    for s in sizes:
        o, x = rand_bits(rng, s, 0.1)
        olds.append(o)
        news.append(x)
    idx, val, nnz, offs = oracle_mod.diff_many(olds, news)
    assert offs[0] == 0 and np.all(np.diff(offs) == nnz)
    for p, (o, x) in enumerate(zip(olds, news)):
        i1, v1 = oracle_mod.diff(o, x)
        assert nnz[p] == i1.size
        assert np.array_equal(idx[offs[p]:offs[p + 1]], i1)
        assert np.array_equal(val[offs[p]:offs[p + 1]], v1)
    # capacity smaller than the total: true counts, truncated payload
    cap = int(offs[-1]) // 2
    idx2, val2, nnz2, offs2 = oracle_mod.diff_many(olds, news, capacity=cap)
    assert np.array_equal(nnz2, nnz) and np.array_equal(offs2, offs)
    assert np.array_equal(idx2, idx[:cap]) and np.array_equal(val2, val[:cap])


# ----------------------------------------------------------------------------
# bf16 rounding and the absorption rule
# ----------------------------------------------------------------------------


def test_bf16_rne_textbook_cases(oracle_mod):
    r = oracle_mod.bf16_rne
    assert r(1.0) == 0x3F80 and r(-2.0) == 0xC000
    assert r(1 + 2 ** -8) == 0x3F80          # tie, even stays
    assert r(1 + 3 * 2 ** -8) == 0x3F82      # tie, odd rounds up to even
    assert r(1 + 2 ** -8 + 2 ** -20) == 0x3F81
    assert r(2 - 2 ** -9) == 0x4000          # tie at binade top carries
    assert r(2.0 ** -133) == 0x0001 and r(2.0 ** -134) == 0x0000
    assert r(-(2.0 ** -134)) == 0x8000       # rounds to zero keeps the sign
    assert r(3 * 2.0 ** -134) == 0x0002      # subnormal tie to even
    max_f = (2 - 2 ** -7) * 2.0 ** 127
    assert r(max_f) == 0x7F7F
    assert r(max_f + 2.0 ** 119) == 0x7F80   # max + half spacing -> inf
    assert r(max_f + 2.0 ** 118) == 0x7F7F
    assert r(float("inf")) == 0x7F80 and r(float("-inf")) == 0xFF80
    assert r(0.0) == 0 and r(-0.0) == 0x8000


def test_bf16_rne_matches_torch_cast(oracle_mod):
    """Library cross-check: torch's float32 -> bfloat16 cast is round to
    nearest even; compare on random float32 patterns plus ties and edges."""
    rng = np.random.default_rng(21)
    u = rng.integers(0, 1 << 32, size=400_000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 1 << 16, size=50_000, dtype=np.uint32) << 16) | 0x8000
    edges = np.array([0, 0x80000000, 0x7F7FFFFF, 0xFF7FFFFF, 0x00000001, 0x007FFFFF,
                      0x00800000, 0x7F800000, 0xFF800000, 0x3F808000, 0x3F818000,
                      0x7F7F8000, 0x7F7F7FFF, 0x00008000, 0x00018000], dtype=np.uint32)
    bits = np.concatenate([u, ties.astype(np.uint32), edges])
    f32 = bits.view(np.float32)
    finite = ~np.isnan(f32)
    f32 = f32[finite]
    want = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy()
    got = oracle_mod.bf16_rne_array(f32.astype(np.float64))
    assert np.array_equal(got, want.view(np.uint16))


ABSORB_K = (0.25, 0.49, 0.5, 0.51, 0.75, 1.0, 1.49)


def _motion_spacing(bits, dw_negative):
    """Spacing of bf16 values next to w on the side the update moves toward."""
    sign = (bits >> 15) & 1
    e = ((bits >> 7) & 0xFF).astype(np.int64)
    mant = bits & 0x7F
    s = np.where(e == 0, 2.0 ** -133, np.ldexp(1.0, (e - 127 - 7).astype(np.int32)))
    toward_zero = (sign == 1) != dw_negative     # update sign opposite to w's sign
    finer_below = toward_zero & (mant == 0) & (e > 1)
    return np.where(finer_below, s / 2, s)


@pytest.mark.parametrize("dw_negative", [False, True])
def test_absorption_bruteforce_all_finite_bf16(oracle_mod, dw_negative):
    """TRL section 2: an update below half the bf16 spacing at w is absorbed by
    the cast and one above it is not (a tie rounds to even).  Checked for every
    one of the 65,280 finite bf16 values and several multiples of the spacing.

    Signed zero is the one exception bitwise: moving +0 downward (or -0 upward)
    by any amount gives the other zero or a nonzero value, so it always changes.
    """
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((allb >> 7) & 0xFF) != 0xFF
    w_bits = allb[finite]
    assert w_bits.size == 65280
    w = bf16_bits_to_f64(w_bits)
    s = _motion_spacing(w_bits, dw_negative)
    mant_odd = (w_bits & 1) == 1
    is_zero = (w_bits & 0x7FFF) == 0
    zero_opposite = is_zero & (((w_bits >> 15) == 1) != dw_negative)
    for k in ABSORB_K:
        dw = -k * s if dw_negative else k * s
        new_bits = oracle_mod.bf16_rne_array(w + dw)
        idx, _ = oracle_mod.diff(w_bits, new_bits)
        changed = np.zeros(w_bits.size, dtype=bool)
        changed[idx] = True
        expect = (k > 0.5) | ((k == 0.5) & mant_odd) | zero_opposite
        bad = np.flatnonzero(changed != expect)
        assert bad.size == 0, (k, [hex(int(b)) for b in w_bits[bad[:8]]])


# ----------------------------------------------------------------------------
# cost-model helper and the synthetic generators
# ----------------------------------------------------------------------------


def test_touched_lines_bruteforce(oracle_mod):
    rng = np.random.default_rng(13)
    for base in (0, 2, 64, 126):
        idx = np.sort(rng.choice(100_000, size=3000, replace=False)).astype(np.int32)
        want = len({(base + 2 * int(i)) // 128 for i in idx})
        assert oracle_mod.touched_lines(idx, 128, base) == want
        want64 = len({(base + 2 * int(i)) // 64 for i in idx})
        assert oracle_mod.touched_lines(idx, 64, base) == want64


@pytest.mark.parametrize("pattern", ["uniform", "clustered"])
@pytest.mark.parametrize("di,frac", list(enumerate(workloads.DENSITIES)))
def test_density_case_exact_count(oracle_mod, pattern, di, frac):
    """Density sweep: the seeded subset is forced to another bf16 value, so the
    diff finds exactly k = round(f*n) changes (runs*2048 when clustered)."""
    n = 1 << 20
    old, new, k = workloads.density_case(n, frac, pattern, di)
    idx, val = oracle_mod.diff(workloads.bits_numpy(old), workloads.bits_numpy(new))
    assert idx.size == k
    if pattern == "clustered":
        assert k % workloads.CLUSTER_RUN == 0
        runs = np.unique(idx // workloads.CLUSTER_RUN)
        assert runs.size * workloads.CLUSTER_RUN == k


def test_step_pair_matches_rne_of_exact_step(oracle_mod):
    """The generators' last step is torch's float32 -> bf16 cast; rounding the
    same float32 intermediate with the oracle's RNE gives the generator's bits
    (both readings of the step)."""
    n = 20_000
    g = torch.Generator()
    for mode in ("bf16_resident", "fp32_master"):
        old, new = workloads.make_step_pair(n, 123, 124, 1e-5, mode)
        w = torch.randn(n, generator=g.manual_seed(123), dtype=torch.float32).mul_(0.02)
        u = torch.randn(n, generator=g.manual_seed(124), dtype=torch.float32)
        assert np.array_equal(oracle_mod.bf16_rne_array(w.double().numpy()),
                              workloads.bits_numpy(old))
        base = old.float() if mode == "bf16_resident" else w
        x32 = base.sub(u, alpha=1e-5)
        assert np.array_equal(oracle_mod.bf16_rne_array(x32.double().numpy()),
                              workloads.bits_numpy(new))


# ----------------------------------------------------------------------------
# sharded diff (VERL code-snippet section `shard_delta_indices`; spec.py
# `derive_placement`)
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("rows", [1, 7, 10, 64, 1000, 1003])
@pytest.mark.parametrize("world", [1, 2, 3, 8, 16])
def test_shard0_rows_match_torch_placement(oracle_mod, rows, world):
    """The row split is torch's own Shard(0) size/offset rule."""
    from torch.distributed.tensor.placement_types import Shard

    for rank in range(world):
        size, first = Shard.local_shard_size_and_offset(rows, world, rank)
        assert oracle_mod.shard0_rows(rows, world, rank) == (first, size)


def test_shard0_flat_offset_is_row_major_index(oracle_mod):
    """The flat offset of a row is numpy's row-major index of [row, 0, ...]."""
    for shape in [(10, 3), (7, 4, 5), (3, 1, 2, 9), (1000, 4096)]:
        for row in range(0, shape[0], max(1, shape[0] // 5)):
            want = int(np.ravel_multi_index((row,) + (0,) * (len(shape) - 1), shape))
            assert oracle_mod.shard0_flat_offset(shape, row) == want


@pytest.mark.parametrize("world", [1, 2, 3, 5, 8])
def test_shard_deltas_concatenate_to_the_full_diff(oracle_mod, world):
    """Every rank diffs only its Shard(0) rows; in rank order the global
    positions and values are exactly the whole tensor's diff."""
    rng = np.random.default_rng(world)
    shapes = [(1003, 37), (64, 128), (5, 3, 7)]
    olds, news = [], []
    for sh in shapes:
        o, x = rand_bits(rng, int(np.prod(sh)), 0.05, special=True)
        olds.append(o)
        news.append(x)
    per_param = {p: ([], []) for p in range(len(shapes))}
    for rank in range(world):
        lo_list, ln_list, offs = [], [], []
        for p, sh in enumerate(shapes):
            first, count = oracle_mod.shard0_rows(sh[0], world, rank)
            inner = int(np.prod(sh[1:]))
            lo_list.append(olds[p][first * inner:(first + count) * inner])
            ln_list.append(news[p][first * inner:(first + count) * inner])
            offs.append(oracle_mod.shard0_flat_offset(sh, first))
        gi, gv, nnz, off = oracle_mod.shard_delta_many(lo_list, ln_list, offs)
        for p in range(len(shapes)):
            per_param[p][0].append(gi[off[p]:off[p + 1]])
            per_param[p][1].append(gv[off[p]:off[p + 1]])
    for p in range(len(shapes)):
        want = np.flatnonzero(olds[p].view(np.int16) != news[p].view(np.int16))
        got_i = np.concatenate(per_param[p][0])
        got_v = np.concatenate(per_param[p][1])
        assert got_i.dtype == np.int64
        assert np.array_equal(got_i, want)
        assert np.array_equal(got_v, news[p][want])


def test_shard_delta_offsets_past_int32(oracle_mod):
    """A shard deep inside a huge parameter: positions past 2^31 are exact."""
    rng = np.random.default_rng(9)
    o, x = rand_bits(rng, 5000, 0.1)
    base = (1 << 31) + 12345
    gi, gv, nnz, off = oracle_mod.shard_delta_many([o, o], [x, x], [base, 3 * (1 << 32)])
    local = np.flatnonzero(o != x)
    assert gi.tolist() == [base + int(i) for i in local] + [3 * (1 << 32) + int(i) for i in local]
    assert int(off[2]) == 2 * local.size


def test_shard_delta_offset_zero_is_diff_many(oracle_mod):
    rng = np.random.default_rng(4)
    olds, news = zip(*[rand_bits(rng, s, 0.03) for s in (100, 0, 4097, 65)])
    gi, gv, nnz, off = oracle_mod.shard_delta_many(olds, news, [0, 0, 0, 0])
    ri, rv, rn, ro = oracle_mod.diff_many(olds, news)
    assert np.array_equal(gi, ri.astype(np.int64))
    assert np.array_equal(gv, rv) and np.array_equal(nnz, rn) and np.array_equal(off, ro)


def test_shard_delta_rejects_negative_offset(oracle_mod):
    a = np.zeros(4, dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle_mod.shard_delta_many([a], [a], [-1])


# ----------------------------------------------------------------------------
# wire encoding (VERL encode.py: DeltaParam pos_width, DeltaFlush, checksum)
# ----------------------------------------------------------------------------


def _wire_case(seed):
    rng = np.random.default_rng(seed)
    numels = [5, 65536, 65537, 100_000, 1, 0, 3000, 65535]
    olds, news = zip(*[rand_bits(rng, n, 0.3) for n in numels])
    ri, rv, rn, ro = oracle_diff_many_np(olds, news)
    return numels, ri, rv, ro


def oracle_diff_many_np(olds, news):
    """The batched delta written with numpy alone (no oracle)."""
    idx, val, nnz = [], [], []
    for o, x in zip(olds, news):
        d = np.flatnonzero(o != x)
        idx.append(d.astype(np.int32))
        val.append(x[d])
        nnz.append(d.size)
    offsets = np.concatenate([[0], np.cumsum(nnz)]).astype(np.int64)
    return np.concatenate(idx), np.concatenate(val), np.array(nnz), offsets


def test_wire_width_reading(oracle_mod):
    assert [oracle_mod.wire_width(n) for n in (0, 1, 65535, 65536, 65537, 1 << 31)] == \
        [2, 2, 2, 2, 4, 4]


def test_wire_encode_matches_numpy_bytes(oracle_mod):
    numels, ri, rv, ro = _wire_case(1)
    pos, po = oracle_mod.wire_encode(ri, ro, numels)
    want, starts = [], [0]
    for p, n in enumerate(numels):
        seg = ri[ro[p]:ro[p + 1]]
        b = seg.astype("<u2" if n <= 65536 else "<u4").tobytes()
        assert seg.size == 0 or int(seg.max()) < n
        want.append(np.frombuffer(b, dtype=np.uint8))
        starts.append(starts[-1] + len(b))
    assert np.array_equal(pos, np.concatenate(want))
    assert po.tolist() == starts
    assert np.array_equal(oracle_mod.wire_decode(pos, po, ro, numels), ri)


def test_hash_bf16_matches_torch_all_patterns(oracle_mod):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    for lo in range(0, 1 << 16, 4096):  # blocks, so one wrong pattern shows
        want = int(torch.hash_tensor(t[lo:lo + 4096]).item())
        assert oracle_mod.hash_bf16(bits[lo:lo + 4096]) == want, hex(lo)
    for b in (0x7F81, 0xFFC1, 0x0001, 0x8000, 0x7F80):  # single patterns: sNaN, qNaN, sub, -0, inf
        one = torch.tensor([b], dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
        assert oracle_mod.hash_bf16(np.array([b], dtype=np.uint16)) == int(torch.hash_tensor(one).item())


def test_hash_bytes_and_checksum_match_torch(oracle_mod):
    numels, ri, rv, ro = _wire_case(2)
    pos, po = oracle_mod.wire_encode(ri, ro, numels)
    tp = torch.from_numpy(pos.copy())
    tv = torch.from_numpy(rv.view(np.int16).copy()).view(torch.bfloat16)
    p = int(torch.hash_tensor(tp).item()) if tp.numel() else 0
    v = int(torch.hash_tensor(tv).item()) if tv.numel() else 0
    assert oracle_mod.hash_bytes(pos) == p
    assert oracle_mod.hash_bf16(rv) == v
    assert oracle_mod.wire_checksum(pos, rv) == p ^ (v << 1)
    # a flipped bit anywhere changes it
    pos2 = pos.copy()
    pos2[len(pos2) // 2] ^= 4
    assert oracle_mod.wire_checksum(pos2, rv) != oracle_mod.wire_checksum(pos, rv)


# ----------------------------------------------------------------------------
# blocked positions: 2 bytes per position for any parameter size
# ----------------------------------------------------------------------------


def test_golden_wire_blocked(oracle_mod):
    g = read_golden("wire_blocked.txt")
    numels = [int(x) for x in g["numels"].split(",")]
    idx = np.array([int(x) for x in g["positions"].split(",")], dtype=np.int32)
    offsets = np.array([int(x) for x in g["offsets"].split(",")], dtype=np.int64)
    want = bytes.fromhex(g["bytes_hex"].replace(" ", ""))
    assert len(want) == int(g["size"])
    got = oracle_mod.wire_encode_blocked(idx, offsets, numels)
    assert got.tobytes() == want
    assert oracle_mod.wire_blocked_size(numels, idx.size) == int(g["size"])
    assert np.array_equal(oracle_mod.wire_decode_blocked(got, offsets, numels), idx)


def _blocked_numpy(idx, offsets, numels):
    """The same bytes from numpy alone: each block's base by a binary search
    of its first element in the parameter's indices, offsets as '<u2'."""
    tables, lows = [], []
    for p, n in enumerate(numels):
        seg = idx[offsets[p]:offsets[p + 1]].astype(np.int64)
        nb = (n + 65535) // 65536
        tables.append(np.searchsorted(seg, np.arange(nb, dtype=np.int64) * 65536)
                      .astype("<u4").tobytes())
        lows.append((seg & 0xFFFF).astype("<u2").tobytes())
    return np.frombuffer(b"".join(tables) + b"".join(lows), dtype=np.uint8)


@pytest.mark.parametrize("seed,frac", [(3, 0.001), (4, 0.03), (5, 0.5), (6, 1.0)])
def test_wire_blocked_matches_numpy_and_round_trips(oracle_mod, seed, frac):
    rng = np.random.default_rng(seed)
    numels = [5, 65536, 65537, 300_001, 1, 0, 3000, 131072, 65535, 200_000]
    olds, news = zip(*[rand_bits(rng, n, frac) for n in numels])
    ri, rv, rn, ro = oracle_diff_many_np(olds, news)
    got = oracle_mod.wire_encode_blocked(ri, ro, numels)
    assert np.array_equal(got, _blocked_numpy(ri, ro, numels))
    blocks = sum((n + 65535) // 65536 for n in numels)
    assert got.size == 4 * blocks + 2 * ri.size == oracle_mod.wire_blocked_size(numels, ri.size)
    assert np.array_equal(oracle_mod.wire_decode_blocked(got, ro, numels), ri)


def test_wire_blocked_rejects_bad_input(oracle_mod):
    numels = [200_000]
    idx = np.array([5, 70_000, 140_000], dtype=np.int32)
    off = np.array([0, 3], dtype=np.int64)
    good = oracle_mod.wire_encode_blocked(idx, off, numels)
    with pytest.raises(ValueError):  # too few bytes
        oracle_mod.wire_decode_blocked(good[:-1], off, numels)
    bad = good.copy()
    bad[4] = 9  # the second block's base above the entry count
    with pytest.raises(ValueError):
        oracle_mod.wire_decode_blocked(bad, off, numels)
    bad = good.copy()
    bad[0] = 1  # the first block's base must be 0
    with pytest.raises(ValueError):
        oracle_mod.wire_decode_blocked(bad, off, numels)
    with pytest.raises(ValueError):  # unsorted or out-of-range indices
        oracle_mod.wire_encode_blocked(np.array([70_000, 5], dtype=np.int32), np.array([0, 2]),
                                       numels)
    with pytest.raises(ValueError):
        oracle_mod.wire_encode_blocked(np.array([200_000], dtype=np.int32), np.array([0, 1]),
                                       numels)
