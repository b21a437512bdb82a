"""Host side of the sharded diff: the Shard(0) placement helpers, checked
against torch's own shard size/offset routine and numpy's row-major index,
and the argument checks of delta_diff_many_sharded (no GPU needed: every
rejected call returns before anything is enqueued)."""
import ctypes

import numpy as np
import pytest

from sparse_bf16_delta_amd import _abi
from sparse_bf16_delta_amd.sharding import flat_offset, shard0_piece


@pytest.mark.parametrize("rows", [0, 1, 7, 10, 64, 1003, 32000])
@pytest.mark.parametrize("world", [1, 2, 3, 8, 16])
def test_shard0_piece_is_torch_shard0(rows, world):
    from torch.distributed.tensor.placement_types import Shard

    covered = 0
    for rank in range(world):
        size, start = Shard.local_shard_size_and_offset(rows, world, rank)
        assert shard0_piece(rows, world, rank) == (start, size)
        covered += size
    assert covered == rows


def test_flat_offset_is_row_major_index():
    for shape in [(10, 3), (7, 4, 5), (32000, 4096), (5,)]:
        for row in range(0, shape[0], max(1, shape[0] // 7)):
            want = int(np.ravel_multi_index((row,) + (0,) * (len(shape) - 1), shape))
            assert flat_offset(shape, row) == want
    assert flat_offset((128256, 16384), 128256 - 1) == (128256 - 1) * 16384  # past 2^31


def test_bad_geometry_raises():
    with pytest.raises(ValueError):
        shard0_piece(10, 0, 0)
    with pytest.raises(ValueError):
        shard0_piece(10, 4, 4)
    with pytest.raises(ValueError):
        flat_offset((10, 3), 11)


def test_sharded_abi_rejects_bad_offsets():
    lib = _abi.load()
    one = ctypes.c_void_p(16)
    ptrs = (ctypes.c_void_p * 1)(16)
    nums = (ctypes.c_int64 * 1)(100)
    neg = (ctypes.c_int64 * 1)(-1)
    big = (ctypes.c_int64 * 1)((1 << 63) - 50)
    ok = (ctypes.c_int64 * 1)(5)
    args = dict(idx=one, val=one, cap=10, nnz=one, off=one, ws=one, wsb=1 << 40)

    def call(fos):
        return lib.delta_diff_many_sharded(1, ptrs, ptrs, nums, fos, args["idx"], args["val"],
                                           args["cap"], args["nnz"], args["off"], args["ws"],
                                           args["wsb"], None)

    assert call(None) == _abi.DELTA_E_INVALID
    assert "flat_offsets is null" in lib.delta_last_error().decode()
    assert call(neg) == _abi.DELTA_E_INVALID
    assert "< 0" in lib.delta_last_error().decode()
    assert call(big) == _abi.DELTA_E_RANGE
    assert "overflows int64" in lib.delta_last_error().decode()
    # a valid offset passes validation and then fails on the too-small workspace
    args["wsb"] = 1
    assert call(ok) == _abi.DELTA_E_WORKSPACE


def test_streamed_abi_rejects_bad_chunks():
    """Every check of delta_apply_streamed fires before any GPU call."""
    lib = _abi.load()
    snaps = (ctypes.c_void_p * 3)(16, 32, 48)
    nums = (ctypes.c_int64 * 3)(10, 20, 30)
    idx = (ctypes.c_int32 * 4)(1, 2, 3, 4)
    val = (ctypes.c_uint16 * 4)(1, 2, 3, 4)
    good = (ctypes.c_int64 * 3)(0, 2, 4)
    not0 = (ctypes.c_int64 * 3)(1, 2, 4)
    dec = (ctypes.c_int64 * 3)(0, 3, 2)

    def chunk(first, count, offs):
        return _abi.HostChunk(first, count, ctypes.addressof(idx), ctypes.addressof(val),
                              ctypes.addressof(offs))

    def call(chs, staging_bytes=1 << 40):
        arr = (_abi.HostChunk * len(chs))(*chs)
        return lib.delta_apply_streamed(3, snaps, nums, len(chs), arr, ctypes.c_void_p(256),
                                        staging_bytes, None, None)

    assert call([chunk(2, 2, good)]) == _abi.DELTA_E_INVALID  # beyond the list
    assert "outside the list" in lib.delta_last_error().decode()
    assert call([chunk(0, 2, not0)]) == _abi.DELTA_E_INVALID
    assert "not from 0" in lib.delta_last_error().decode()
    assert call([chunk(0, 2, dec)]) == _abi.DELTA_E_INVALID
    assert "decrease" in lib.delta_last_error().decode()
    assert call([chunk(0, 2, good)], staging_bytes=16) == _abi.DELTA_E_WORKSPACE
    # a parameter list without its arrays is rejected even with no chunks
    assert lib.delta_apply_streamed(3, None, None, 0, None, ctypes.c_void_p(256), 1 << 40,
                                    None, None) == _abi.DELTA_E_INVALID
    assert "null argument" in lib.delta_last_error().decode()
    assert lib.xor_apply_streamed(None, None, 10, 0, None, 0, None, None) == _abi.DELTA_E_INVALID
    assert lib.xor_apply_streamed(ctypes.c_void_p(16), ctypes.c_void_p(16), 100, 64,
                                  ctypes.c_void_p(256), 8, None, None) == _abi.DELTA_E_WORKSPACE
    assert lib.delta_streamed_staging_size(-1, 1, 0, 0) == 0
    assert lib.xor_streamed_staging_size(0) == 0
    # counts whose staging would not fit size_t are refused, not wrapped
    huge = (ctypes.c_int64 * 3)(0, 2, 1 << 62)
    assert call([chunk(0, 2, huge)]) == _abi.DELTA_E_RANGE
    assert "more than a staging buffer" in lib.delta_last_error().decode()
    assert lib.delta_streamed_staging_size(3, 1, 2, 1 << 62) == 0
    assert lib.delta_streamed_staging_size(3, 1, 2, 1000) > 0
    assert lib.xor_streamed_staging_size(1 << 62) == 0
    assert lib.xor_apply_streamed(ctypes.c_void_p(16), ctypes.c_void_p(16), 100, 1 << 62,
                                  ctypes.c_void_p(256), 1 << 40, None, None) == _abi.DELTA_E_RANGE


def test_host_apply_abi_rejects_bad_arguments():
    """delta_apply_many_host checks its counts, pointers, sizes and offsets
    before it asks the runtime about the host buffers or launches anything."""
    lib = _abi.load()
    snaps = (ctypes.c_void_p * 2)(16, 32)
    nums = (ctypes.c_int64 * 2)(10, 20)
    idx = (ctypes.c_int32 * 4)(1, 2, 3, 4)
    val = (ctypes.c_uint16 * 4)(1, 2, 3, 4)
    ws = ctypes.c_void_p(256)

    def call(offs, n=2, sp=snaps, nm=nums, max_nnz=4):
        return lib.delta_apply_many_host(n, sp, nm, ctypes.addressof(idx), ctypes.addressof(val),
                                         offs, max_nnz, None, ws, 1 << 30, None)

    good = (ctypes.c_int64 * 3)(0, 2, 4)
    assert call(good, n=-1) == _abi.DELTA_E_INVALID
    assert call(good, max_nnz=-1) == _abi.DELTA_E_INVALID
    assert call(None) == _abi.DELTA_E_INVALID
    assert call(good, sp=None) == _abi.DELTA_E_INVALID
    assert call(good, nm=(ctypes.c_int64 * 2)(10, -5)) == _abi.DELTA_E_INVALID
    assert call(good, nm=(ctypes.c_int64 * 2)(10, 1 << 31)) == _abi.DELTA_E_RANGE
    assert call(good, sp=(ctypes.c_void_p * 2)(16, None)) == _abi.DELTA_E_INVALID
    assert "null snapshot" in lib.delta_last_error().decode()
    assert call((ctypes.c_int64 * 3)(1, 2, 4)) == _abi.DELTA_E_INVALID
    assert "offsets[0]" in lib.delta_last_error().decode()
    assert call((ctypes.c_int64 * 3)(0, 3, 2)) == _abi.DELTA_E_INVALID
    assert "decrease" in lib.delta_last_error().decode()
    # a count above 2^62 is refused; one of 2^62, whose int32 bytes wrap 64 bits,
    # never passes the pinned-range check
    huge = (1 << 62) + 4
    assert call((ctypes.c_int64 * 3)(0, 2, huge), max_nnz=huge) == _abi.DELTA_E_RANGE
    edge = 1 << 62
    assert call((ctypes.c_int64 * 3)(0, 2, edge), max_nnz=edge) == _abi.DELTA_E_INVALID
    assert "pinned host memory" in lib.delta_last_error().decode()


def test_wire_abi_rejects_bad_arguments():
    lib = _abi.load()
    one = ctypes.c_void_p(16)
    nums = (ctypes.c_int64 * 2)(10, -1)
    assert lib.delta_wire_encode(2, nums, one, one, 5, one, 10, one, one, 1 << 30, None) == \
        _abi.DELTA_E_INVALID
    assert "numels[1]" in lib.delta_last_error().decode()
    big = (ctypes.c_int64 * 1)(1 << 31)
    assert lib.delta_wire_decode(1, big, one, 8, one, one, 5, one, None, one, 1 << 30, None) == \
        _abi.DELTA_E_RANGE
    assert lib.delta_wire_decode(1, nums, one, -1, one, one, 5, one, None, one, 1 << 30,
                                 None) == _abi.DELTA_E_INVALID
    assert lib.delta_wire_decode(1, nums, None, 8, one, one, 5, one, None, one, 1 << 30,
                                 None) == _abi.DELTA_E_INVALID
    ok = (ctypes.c_int64 * 1)(10)
    assert lib.delta_wire_encode(1, ok, one, one, 5, one, 10, one, one, 1, None) == \
        _abi.DELTA_E_WORKSPACE
    assert lib.delta_wire_hash(None, 4, None, 0, one, None) == _abi.DELTA_E_INVALID
    assert lib.delta_wire_hash(one, -1, one, 0, one, None) == _abi.DELTA_E_INVALID
    # positions move as 2-byte halves: an odd address is rejected before any launch
    odd = ctypes.c_void_p(17)
    assert lib.delta_wire_encode(1, ok, one, one, 5, odd, 10, one, one, 1 << 30, None) == \
        _abi.DELTA_E_INVALID
    assert "2-byte aligned" in lib.delta_last_error().decode()
    assert lib.delta_wire_decode(1, ok, odd, 8, one, one, 5, one, None, one, 1 << 30,
                                 None) == _abi.DELTA_E_INVALID
    assert "2-byte aligned" in lib.delta_last_error().decode()


def test_wire_sizes_are_the_library_rule():
    """The byte counts a caller needs come from the library, from the widths
    and block tables that the oracle pins (the binding holds no width rule)."""
    lib = _abi.load()
    numels = [5, 65536, 65537, 300_001, 0]
    nums = (ctypes.c_int64 * len(numels))(*numels)
    off = (ctypes.c_int64 * 6)(0, 3, 10, 12, 20, 20)
    counts = [3, 7, 2, 8, 0]
    from oracle import oracle as o

    want = sum(c * o.wire_width(n) for c, n in zip(counts, numels))
    assert lib.delta_wire_positions_size(len(numels), nums, off) == want
    assert lib.delta_wire_blocked_size(len(numels), nums, 20) == o.wire_blocked_size(numels, 20)
    assert lib.delta_wire_blocked_size(len(numels), nums, 20) == 4 * (1 + 1 + 2 + 5 + 0) + 40
    bad = (ctypes.c_int64 * 6)(0, 3, 2, 12, 20, 20)
    assert lib.delta_wire_positions_size(len(numels), nums, bad) == -1
    assert lib.delta_wire_blocked_size(-1, nums, 0) == -1
    # sizes past int64 are reported as -1, not wrapped
    top = (1 << 63) - 1
    assert lib.delta_wire_blocked_size(len(numels), nums, top) == -1
    assert lib.delta_wire_blocked_size(len(numels), nums, (top - 36) // 2) == top - 1
    wide = (ctypes.c_int64 * 6)(0, 0, 0, 0, (1 << 62) - 1, (1 << 62) - 1)  # 4 bytes each
    assert lib.delta_wire_positions_size(len(numels), nums, wide) == -1
    neg = (ctypes.c_int64 * 6)(-5, 3, 10, 12, 20, 20)
    assert lib.delta_wire_positions_size(len(numels), nums, neg) == -1


def test_blocked_wire_abi_rejects_bad_arguments():
    lib = _abi.load()
    one = ctypes.c_void_p(16)
    nums = (ctypes.c_int64 * 1)(200_000)  # 4 blocks: 16 bytes of tables
    assert lib.delta_wire_encode_blocked(1, nums, one, one, -1, one, 8, one, 1 << 30,
                                         None) == _abi.DELTA_E_INVALID
    assert lib.delta_wire_encode_blocked(1, nums, one, one, 5, ctypes.c_void_p(18), 8, one,
                                         1 << 30, None) == _abi.DELTA_E_INVALID
    assert "aligned" in lib.delta_last_error().decode()
    assert lib.delta_wire_encode_blocked(1, nums, one, one, 5, one, 8, one, 1, None) == \
        _abi.DELTA_E_WORKSPACE
    # fewer bytes than the block tables: rejected before anything is read
    assert lib.delta_wire_decode_blocked(1, nums, one, 12, one, 5, one, None, one, 1 << 30,
                                         None) == _abi.DELTA_E_INVALID
    assert "block bases" in lib.delta_last_error().decode()
    big = (ctypes.c_int64 * 1)(1 << 31)
    assert lib.delta_wire_decode_blocked(1, big, one, 1 << 20, one, 5, one, None, one, 1 << 30,
                                         None) == _abi.DELTA_E_RANGE
