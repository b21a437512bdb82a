"""GPU parity of the wire encoding: positions byte block, decode and the
flush hashes, against the oracle, bit for bit."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sbd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_bf16_delta_amd as m

    m.load()
    return m


def np_bits(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)


def delta_case(seed, numels, frac):
    rng = np.random.default_rng(seed)
    olds, news = [], []
    for n in numels:
        o = rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
        x = o.copy()
        k = int(round(frac * n))
        if k:
            pos = rng.choice(n, size=k, replace=False)
            x[pos] = (o[pos].astype(np.uint32) + rng.integers(1, 1 << 16, size=k)).astype(np.uint16)
        olds.append(o)
        news.append(x)
    return olds, news


NUMELS = [5, 65536, 65537, 100_000, 1, 0, 3000, 65535, 3, 200_003]


@pytest.mark.parametrize("frac", [0.0, 0.01, 0.3, 1.0])
def test_wire_encode_decode_hash_match_oracle(sbd, oracle_mod, frac):
    olds, news = delta_case(int(frac * 100), NUMELS, frac)
    ri, rv, rn, ro = oracle_mod.diff_many(olds, news)
    want_pos, want_po = oracle_mod.wire_encode(ri, ro, NUMELS)
    gi, gv, gn, go = sbd.diff_many([torch.from_numpy(o.view(np.int16)).cuda() for o in olds],
                                   [torch.from_numpy(x.view(np.int16)).cuda() for x in news])
    pos, po = sbd.wire_encode(gi, go, NUMELS)
    assert np.array_equal(po.cpu().numpy(), want_po)
    assert np.array_equal(pos.cpu().numpy(), want_pos)
    back = sbd.wire_decode(pos, po, go, NUMELS)
    assert np.array_equal(back.cpu().numpy(), ri)
    hp, hv = sbd.wire_hashes(pos, gv)
    assert hp == oracle_mod.hash_bytes(want_pos)
    assert hv == oracle_mod.hash_bf16(rv)
    assert sbd.wire_checksum(pos, gv) == oracle_mod.wire_checksum(want_pos, rv)


def test_wire_hash_every_bf16_pattern_and_unaligned_bytes(sbd, oracle_mod):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = torch.from_numpy(bits.view(np.int16).copy()).cuda()
    rng = np.random.default_rng(3)
    raw = rng.integers(0, 256, size=100_003, dtype=np.uint8)
    buf = torch.from_numpy(raw).cuda()
    for off in (0, 1, 7, 16):  # unaligned starts use the byte path
        for n in (0, 1, 15, 16, 17, 100_003 - off):
            hp, hv = sbd.wire_hashes(buf[off:off + n], vals)
            assert hp == oracle_mod.hash_bytes(raw[off:off + n])
            assert hv == oracle_mod.hash_bf16(bits)


def test_wire_encode_respects_capacity(sbd, oracle_mod):
    import ctypes
    from sparse_bf16_delta_amd import _abi
    from sparse_bf16_delta_amd.ops import _ptr, _stream

    olds, news = delta_case(9, NUMELS, 0.2)
    ri, rv, rn, ro = oracle_mod.diff_many(olds, news)
    want_pos, want_po = oracle_mod.wire_encode(ri, ro, NUMELS)
    idx = torch.from_numpy(ri).cuda()
    off = torch.from_numpy(ro).cuda()
    cut = int(want_po[3]) + 6  # inside the fourth parameter's positions
    guard = 512
    pos = torch.full((cut + guard,), 0xAB, dtype=torch.uint8, device="cuda")
    po = torch.empty(len(NUMELS) + 1, dtype=torch.int64, device="cuda")
    lib = _abi.load()
    ws = torch.empty(lib.delta_workspace_size(0, len(NUMELS)), dtype=torch.uint8, device="cuda")
    nums = (ctypes.c_int64 * len(NUMELS))(*NUMELS)
    _abi.check(lib.delta_wire_encode(len(NUMELS), nums, _ptr(idx), _ptr(off), ri.size, _ptr(pos),
                                     cut, _ptr(po), _ptr(ws), ws.numel(), _stream(idx.device)))
    got = pos.cpu().numpy()
    whole = int(want_po[3]) + 4  # the fourth parameter is 4 bytes wide: one whole entry fits
    assert np.array_equal(got[:whole], want_pos[:whole])
    assert np.all(got[whole:] == 0xAB)  # the entry across the cut and all past it: untouched
    assert np.array_equal(po.cpu().numpy(), want_po)  # the true sizes


def test_wire_wrappers_reject_bad_arguments(sbd):
    """dtype, device and length mistakes raise before anything is launched."""
    idx = torch.arange(4, dtype=torch.int32, device="cuda")
    off = torch.tensor([0, 4], dtype=torch.int64, device="cuda")
    with pytest.raises(ValueError):
        sbd.wire_encode(idx.long(), off, [10])
    with pytest.raises(ValueError):
        sbd.wire_encode(idx, off.cpu(), [10])
    with pytest.raises(ValueError):
        sbd.wire_encode(idx, off, [10, 20])
    pos, po = sbd.wire_encode(idx, off, [10])
    with pytest.raises(ValueError):
        sbd.wire_decode(pos.view(torch.int8), po, off, [10])
    with pytest.raises(ValueError):
        sbd.wire_decode(pos, po.int(), off, [10])
    with pytest.raises(ValueError):
        sbd.wire_decode(pos, po, off.cpu(), [10])
    assert torch.equal(sbd.wire_decode(pos, po, off, [10]), idx)


def test_wire_decode_untrusted_block(sbd, oracle_mod):
    """A received positions block that is truncated, or whose parameter spans
    do not match the counts, is read only inside its bytes: the bad entries
    come back as -1 and are counted (the binding raises)."""
    import ctypes
    from sparse_bf16_delta_amd import _abi
    from sparse_bf16_delta_amd.ops import _ptr, _stream

    olds, news = delta_case(13, NUMELS, 0.05)
    ri, rv, rn, ro = oracle_mod.diff_many(olds, news)
    want_pos, want_po = oracle_mod.wire_encode(ri, ro, NUMELS)
    off = torch.from_numpy(ro).cuda()
    lib = _abi.load()
    ws = torch.empty(lib.delta_workspace_size(0, len(NUMELS)), dtype=torch.uint8, device="cuda")
    nums = (ctypes.c_int64 * len(NUMELS))(*NUMELS)
    k = len(NUMELS)

    def decode(pos_bytes, po, nbytes):
        pos = torch.from_numpy(pos_bytes.copy()).cuda()
        pot = torch.from_numpy(np.asarray(po, dtype=np.int64).copy()).cuda()
        idx = torch.full((ri.size,), 77, dtype=torch.int32, device="cuda")
        v = torch.full((1,), -1, dtype=torch.int64, device="cuda")
        _abi.check(lib.delta_wire_decode(k, nums, _ptr(pos), nbytes, _ptr(pot), _ptr(off),
                                         ri.size, _ptr(idx), _ptr(v), _ptr(ws), ws.numel(),
                                         _stream(off.device)))
        return idx.cpu().numpy(), int(v.item())

    got, bad = decode(want_pos, want_po, want_pos.size)
    assert bad == 0 and np.array_equal(got, ri)
    # truncated: the last 10 bytes are missing (the block is 4-byte wide there)
    got, bad = decode(want_pos[:-10], want_po, want_pos.size - 10)
    lost = (10 + 3) // 4  # entries whose bytes reach into the missing tail
    assert bad == lost
    assert np.array_equal(got[:-lost], ri[:-lost]) and np.all(got[-lost:] == -1)
    # a span shifted past the block: parameter 3's start moved beyond the end
    po2 = want_po.copy()
    po2[3] = want_po[-1] + 64
    got, bad = decode(want_pos, po2, want_pos.size)
    n3 = int(ro[4] - ro[3])
    assert bad >= n3 and np.all(got[ro[3]:ro[4]] == -1)
    with pytest.raises(sbd.DeltaError, match="malformed"):
        sbd.wire_decode(torch.from_numpy(want_pos[:-10].copy()).cuda(),
                        torch.from_numpy(want_po).cuda(), off, NUMELS)


BLOCKED_NUMELS = [5, 65536, 65537, 300_001, 1, 0, 3000, 131072, 65535, 200_003, 1 << 22]


@pytest.mark.parametrize("frac", [0.0, 0.001, 0.0118, 0.3, 1.0])
def test_wire_blocked_matches_oracle(sbd, oracle_mod, frac):
    """Blocked positions of a diff_many delta equal the oracle's bytes, decode
    back to the delta, and the flush checksum over them equals the oracle's."""
    olds, news = delta_case(int(frac * 1000) + 3, BLOCKED_NUMELS, frac)
    ri, rv, rn, ro = oracle_mod.diff_many(olds, news)
    want = oracle_mod.wire_encode_blocked(ri, ro, BLOCKED_NUMELS)
    gi, gv, gn, go = sbd.diff_many([torch.from_numpy(o.view(np.int16)).cuda() for o in olds],
                                   [torch.from_numpy(x.view(np.int16)).cuda() for x in news])
    data = sbd.wire_encode_blocked(gi, go, BLOCKED_NUMELS)
    assert np.array_equal(data.cpu().numpy(), want)
    back = sbd.wire_decode_blocked(data, go, BLOCKED_NUMELS)
    assert np.array_equal(back.cpu().numpy(), ri)
    assert sbd.wire_checksum(data, gv) == oracle_mod.wire_checksum(want, rv)
    print(f"frac {frac}: {ri.size} entries, {want.size} bytes "
          f"({want.size / max(ri.size, 1):.3f} per entry)")


def test_wire_blocked_capacity_and_untrusted_bytes(sbd, oracle_mod):
    """Encode writes nothing at or past its capacity; decode of truncated or
    corrupted bytes reads only inside them and counts what is wrong."""
    import ctypes
    from sparse_bf16_delta_amd import _abi
    from sparse_bf16_delta_amd.ops import _ptr, _stream

    olds, news = delta_case(21, BLOCKED_NUMELS, 0.02)
    ri, rv, rn, ro = oracle_mod.diff_many(olds, news)
    want = oracle_mod.wire_encode_blocked(ri, ro, BLOCKED_NUMELS)
    idx = torch.from_numpy(ri).cuda()
    off = torch.from_numpy(ro).cuda()
    lib = _abi.load()
    k = len(BLOCKED_NUMELS)
    nums = (ctypes.c_int64 * k)(*BLOCKED_NUMELS)
    ws = torch.empty(lib.delta_workspace_size(0, k), dtype=torch.uint8, device="cuda")
    cut = want.size - 101
    out = torch.full((want.size + 256,), 0xAB, dtype=torch.uint8, device="cuda")
    _abi.check(lib.delta_wire_encode_blocked(k, nums, _ptr(idx), _ptr(off), ri.size, _ptr(out),
                                             cut, _ptr(ws), ws.numel(), _stream(idx.device)))
    got = out.cpu().numpy()
    assert np.array_equal(got[:cut - 1], want[:cut - 1])  # whole 2-byte offsets below the cut
    assert np.all(got[cut:] == 0xAB)

    def decode(data, nbytes):
        d = torch.from_numpy(data.copy()).cuda()
        res = torch.full((ri.size,), 77, dtype=torch.int32, device="cuda")
        v = torch.full((1,), -1, dtype=torch.int64, device="cuda")
        _abi.check(lib.delta_wire_decode_blocked(k, nums, _ptr(d), nbytes, _ptr(off), ri.size,
                                                 _ptr(res), _ptr(v), _ptr(ws), ws.numel(),
                                                 _stream(off.device)))
        return res.cpu().numpy(), int(v.item())

    res, bad = decode(want, want.size)
    assert bad == 0 and np.array_equal(res, ri)
    res, bad = decode(want[:-6], want.size - 6)  # three offsets missing
    assert bad == 3 and np.all(res[-3:] == -1) and np.array_equal(res[:-3], ri[:-3])
    broken = want.copy()
    broken[4 * 3:4 * 3 + 4] = np.frombuffer(np.uint32(1 << 30).tobytes(), dtype=np.uint8)
    res, bad = decode(broken, broken.size)  # a base far above its parameter's count
    assert bad >= 1
    with pytest.raises(sbd.DeltaError, match="malformed"):
        sbd.wire_decode_blocked(torch.from_numpy(want[:-6].copy()).cuda(), off, BLOCKED_NUMELS)


@pytest.mark.parametrize("in_shift", [0, 4, 8, 12])
@pytest.mark.parametrize("out_shift", [0, 1, 3])
def test_wire_blocked_decode_alignments(sbd, oracle_mod, in_shift, out_shift):
    """Decode reads its bytes and writes its indices at any alignment the
    contract allows: blocks placed 0, 4, 8 or 12 bytes past a 16-byte
    aligned address (the offsets after the tables then start 8- or only
    4-byte aligned), and indices written from 0, 1 or 3 elements past one,
    match the oracle; the elements around the output are untouched."""
    import ctypes
    from sparse_bf16_delta_amd import _abi
    from sparse_bf16_delta_amd.ops import _ptr, _stream

    # 2 + 1 + 1 + 3 + 1 = 8 blocks, or 9 with the last parameter: the block
    # tables end 8- or 4-byte aligned relative to the start
    numels = [70_000, 3, 65536, 131_073, 9] + ([100] if out_shift == 1 else [])
    olds, news = delta_case(31 + in_shift + 7 * out_shift, numels, 0.05)
    ri, rv, rn, ro = oracle_mod.diff_many(olds, news)
    want = oracle_mod.wire_encode_blocked(ri, ro, numels)
    lib = _abi.load()
    k = len(numels)
    nums = (ctypes.c_int64 * k)(*numels)
    ws = torch.empty(lib.delta_workspace_size(0, k), dtype=torch.uint8, device="cuda")
    buf = torch.zeros(want.size + 16, dtype=torch.uint8, device="cuda")
    buf[in_shift:in_shift + want.size] = torch.from_numpy(want).cuda()
    data = buf[in_shift:in_shift + want.size]
    off = torch.from_numpy(ro).cuda()
    res = torch.full((ri.size + 8,), 77, dtype=torch.int32, device="cuda")
    out = res[out_shift:out_shift + ri.size]
    v = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    _abi.check(lib.delta_wire_decode_blocked(k, nums, _ptr(data), want.size, _ptr(off), ri.size,
                                             _ptr(out), _ptr(v), _ptr(ws), ws.numel(),
                                             _stream(off.device)))
    got = res.cpu().numpy()
    assert int(v.item()) == 0
    assert np.array_equal(got[out_shift:out_shift + ri.size], ri)
    assert np.all(got[:out_shift] == 77) and np.all(got[out_shift + ri.size:] == 77)


@pytest.mark.parametrize("out_shift", [0, 4, 8, 12])
@pytest.mark.parametrize("idx_shift", [0, 1, 3])
def test_wire_blocked_encode_alignments(sbd, oracle_mod, out_shift, idx_shift):
    """Encode reads indices and writes bytes at any alignment the contract
    allows: indices from 0, 1 or 3 elements past a 16-byte aligned address,
    the block 0, 4, 8 or 12 bytes past one (the offsets after the tables
    then start 8- or only 4-byte aligned); its bytes equal the oracle's and
    the bytes around them are untouched."""
    import ctypes
    from sparse_bf16_delta_amd import _abi
    from sparse_bf16_delta_amd.ops import _ptr, _stream

    numels = [70_000, 3, 65536, 131_073, 9] + ([100] if idx_shift == 1 else [])
    olds, news = delta_case(51 + out_shift + 7 * idx_shift, numels, 0.05)
    ri, rv, rn, ro = oracle_mod.diff_many(olds, news)
    want = oracle_mod.wire_encode_blocked(ri, ro, numels)
    lib = _abi.load()
    k = len(numels)
    nums = (ctypes.c_int64 * k)(*numels)
    ws = torch.empty(lib.delta_workspace_size(0, k), dtype=torch.uint8, device="cuda")
    ibuf = torch.zeros(ri.size + 8, dtype=torch.int32, device="cuda")
    ibuf[idx_shift:idx_shift + ri.size] = torch.from_numpy(ri).cuda()
    idx = ibuf[idx_shift:idx_shift + ri.size]
    off = torch.from_numpy(ro).cuda()
    buf = torch.full((want.size + 32,), 0xAB, dtype=torch.uint8, device="cuda")
    out = buf[out_shift:out_shift + want.size]
    _abi.check(lib.delta_wire_encode_blocked(k, nums, _ptr(idx), _ptr(off), ri.size, _ptr(out),
                                             want.size, _ptr(ws), ws.numel(), _stream(off.device)))
    got = buf.cpu().numpy()
    assert np.array_equal(got[out_shift:out_shift + want.size], want)
    assert np.all(got[:out_shift] == 0xAB) and np.all(got[out_shift + want.size:] == 0xAB)


@pytest.mark.parametrize("shift", [2, 4, 6])
def test_wire_positions_at_shifted_addresses(sbd, oracle_mod, shift):
    """The per-parameter block encoded to, and decoded from, an address 2, 4
    or 6 bytes past a 16-byte aligned one (4-byte positions then move as
    words or as halves): the bytes and the indices equal the oracle's."""
    import ctypes
    from sparse_bf16_delta_amd import _abi
    from sparse_bf16_delta_amd.ops import _ptr, _stream

    olds, news = delta_case(61 + shift, NUMELS, 0.05)
    ri, rv, rn, ro = oracle_mod.diff_many(olds, news)
    want_pos, want_po = oracle_mod.wire_encode(ri, ro, NUMELS)
    lib = _abi.load()
    k = len(NUMELS)
    nums = (ctypes.c_int64 * k)(*NUMELS)
    ws = torch.empty(lib.delta_workspace_size(0, k), dtype=torch.uint8, device="cuda")
    idx = torch.from_numpy(ri).cuda()
    off = torch.from_numpy(ro).cuda()
    po = torch.empty(k + 1, dtype=torch.int64, device="cuda")
    buf = torch.full((want_pos.size + 32,), 0xAB, dtype=torch.uint8, device="cuda")
    pos = buf[shift:shift + want_pos.size]
    _abi.check(lib.delta_wire_encode(k, nums, _ptr(idx), _ptr(off), ri.size, _ptr(pos),
                                     want_pos.size, _ptr(po), _ptr(ws), ws.numel(),
                                     _stream(off.device)))
    got = buf.cpu().numpy()
    assert np.array_equal(po.cpu().numpy(), want_po)
    assert np.array_equal(got[shift:shift + want_pos.size], want_pos)
    assert np.all(got[:shift] == 0xAB) and np.all(got[shift + want_pos.size:] == 0xAB)
    back = torch.full((ri.size,), 77, dtype=torch.int32, device="cuda")
    v = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    _abi.check(lib.delta_wire_decode(k, nums, _ptr(pos), want_pos.size, _ptr(po), _ptr(off),
                                     ri.size, _ptr(back), _ptr(v), _ptr(ws), ws.numel(),
                                     _stream(off.device)))
    assert int(v.item()) == 0
    assert np.array_equal(back.cpu().numpy(), ri)
