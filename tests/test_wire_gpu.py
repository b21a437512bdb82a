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
