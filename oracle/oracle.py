"""ctypes binding for the CPU oracle (``sbd_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use this module; the product library never does.  The oracle
shares no code with the HIP path.  Inputs and outputs are numpy arrays of bf16
bit patterns (``uint16``) and int32 indices; all arithmetic happens in C.

Build: ``python -m oracle.build`` (gcc, single file, no dependencies).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# A mutation check may point this at a deliberately broken build of the oracle.
LIB_PATH = os.environ.get("SBD_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, u16 = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint16
    vp = ctypes.c_void_p
    lib.oracle_diff.argtypes = [vp, vp, i64, vp, vp]
    lib.oracle_diff.restype = i64
    lib.oracle_diff_many.argtypes = [i32, vp, vp, vp, vp, vp, i64, vp, vp]
    lib.oracle_diff_many.restype = ctypes.c_int
    lib.oracle_shard_delta_many.argtypes = [i32, vp, vp, vp, vp, vp, vp, i64, vp, vp]
    lib.oracle_shard_delta_many.restype = ctypes.c_int
    lib.oracle_wire_width.argtypes = [i64]
    lib.oracle_wire_width.restype = ctypes.c_int
    lib.oracle_wire_encode.argtypes = [i32, vp, vp, vp, vp, vp]
    lib.oracle_wire_encode.restype = i64
    lib.oracle_wire_decode.argtypes = [i32, vp, vp, vp, vp, vp]
    lib.oracle_wire_decode.restype = ctypes.c_int
    lib.oracle_wire_blocked_size.argtypes = [i32, vp, i64]
    lib.oracle_wire_blocked_size.restype = i64
    lib.oracle_wire_encode_blocked.argtypes = [i32, vp, vp, vp, vp]
    lib.oracle_wire_encode_blocked.restype = i64
    lib.oracle_wire_decode_blocked.argtypes = [i32, vp, vp, i64, vp, vp]
    lib.oracle_wire_decode_blocked.restype = ctypes.c_int
    lib.oracle_hash_bytes.argtypes = [vp, i64]
    lib.oracle_hash_bytes.restype = ctypes.c_uint64
    lib.oracle_hash_bf16.argtypes = [vp, i64]
    lib.oracle_hash_bf16.restype = ctypes.c_uint64
    lib.oracle_apply.argtypes = [vp, i64, vp, vp, i64]
    lib.oracle_apply.restype = ctypes.c_int
    lib.oracle_xor_mask.argtypes = [vp, vp, vp, i64]
    lib.oracle_xor_mask.restype = None
    lib.oracle_xor_apply.argtypes = [vp, vp, i64]
    lib.oracle_xor_apply.restype = None
    lib.oracle_bf16_rne.argtypes = [ctypes.c_double]
    lib.oracle_bf16_rne.restype = u16
    lib.oracle_bf16_rne_array.argtypes = [vp, vp, i64]
    lib.oracle_bf16_rne_array.restype = None
    lib.oracle_sparsity.argtypes = [i64, i64]
    lib.oracle_sparsity.restype = ctypes.c_double
    lib.oracle_touched_lines.argtypes = [vp, i64, i64, i64]
    lib.oracle_touched_lines.restype = i64
    _lib = lib
    return lib


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected uint16 bit patterns, got {a.dtype}")
    return a.reshape(-1)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def diff(old_bits, new_bits):
    """Bitwise diff + compaction: returns (idx int32, val uint16)."""
    old_bits, new_bits = _u16(old_bits), _u16(new_bits)
    if old_bits.shape != new_bits.shape:
        raise ValueError("old and new differ in size")
    n = old_bits.size
    idx = np.empty(n, dtype=np.int32)
    val = np.empty(n, dtype=np.uint16)
    k = _load().oracle_diff(_ptr(old_bits), _ptr(new_bits), n, _ptr(idx), _ptr(val))
    if k < 0:
        raise ValueError(f"oracle_diff rejected n={n}")
    return idx[:k].copy(), val[:k].copy()


def diff_many(olds, news, capacity=None):
    """Batched diff over a parameter list: (idx_cat, val_cat, nnz[k], offsets[k+1])."""
    olds = [_u16(o) for o in olds]
    news = [_u16(x) for x in news]
    if len(olds) != len(news):
        raise ValueError("parameter lists differ in length")
    k = len(olds)
    numels = np.array([o.size for o in olds], dtype=np.int64)
    for o, x in zip(olds, news):
        if o.size != x.size:
            raise ValueError("old and new differ in size")
    total = int(numels.sum())
    cap = total if capacity is None else int(capacity)
    idx = np.empty(max(cap, 1), dtype=np.int32)
    val = np.empty(max(cap, 1), dtype=np.uint16)
    nnz = np.zeros(k, dtype=np.int64)
    offsets = np.zeros(k + 1, dtype=np.int64)
    optrs = (ctypes.c_void_p * max(k, 1))(*[_ptr(o) for o in olds])
    nptrs = (ctypes.c_void_p * max(k, 1))(*[_ptr(x) for x in news])
    rc = _load().oracle_diff_many(
        k, ctypes.addressof(optrs), ctypes.addressof(nptrs), _ptr(numels),
        _ptr(idx), _ptr(val), cap, _ptr(nnz), _ptr(offsets))
    if rc != 0:
        raise ValueError("oracle_diff_many rejected its arguments")
    m = min(int(offsets[k]), cap)
    return idx[:m].copy(), val[:m].copy(), nnz, offsets


def shard_delta_many(olds, news, flat_offsets, capacity=None):
    """Sharded batched diff: (gidx_cat int64, val_cat, nnz[k], offsets[k+1]),
    gidx = flat_offsets[p] + local index."""
    olds = [_u16(o) for o in olds]
    news = [_u16(x) for x in news]
    if len(olds) != len(news) or len(olds) != len(flat_offsets):
        raise ValueError("parameter lists differ in length")
    k = len(olds)
    numels = np.array([o.size for o in olds], dtype=np.int64)
    for o, x in zip(olds, news):
        if o.size != x.size:
            raise ValueError("old and new differ in size")
    fo = np.ascontiguousarray(flat_offsets, dtype=np.int64)
    total = int(numels.sum())
    cap = total if capacity is None else int(capacity)
    gidx = np.empty(max(cap, 1), dtype=np.int64)
    val = np.empty(max(cap, 1), dtype=np.uint16)
    nnz = np.zeros(k, dtype=np.int64)
    offsets = np.zeros(k + 1, dtype=np.int64)
    optrs = (ctypes.c_void_p * max(k, 1))(*[_ptr(o) for o in olds])
    nptrs = (ctypes.c_void_p * max(k, 1))(*[_ptr(x) for x in news])
    rc = _load().oracle_shard_delta_many(
        k, ctypes.addressof(optrs), ctypes.addressof(nptrs), _ptr(numels), _ptr(fo),
        _ptr(gidx), _ptr(val), cap, _ptr(nnz), _ptr(offsets))
    if rc != 0:
        raise ValueError("oracle_shard_delta_many rejected its arguments")
    m = min(int(offsets[k]), cap)
    return gidx[:m].copy(), val[:m].copy(), nnz, offsets


def shard0_rows(rows: int, world: int, rank: int):
    """(first_row, row_count) of `rank`'s Shard(0) piece of a dimension of
    `rows` rows over `world` ranks: equal pieces of ceil(rows / world) rows,
    the last ones shorter or empty ([VERL] spec.py `derive_placement`, which
    takes the global offset of the FSDP2 Shard(0) placement)."""
    if rows < 0 or world < 1 or not 0 <= rank < world:
        raise ValueError("bad shard geometry")
    piece = (rows + world - 1) // world
    first = min(piece * rank, rows)
    return first, min(piece, rows - first)


def shard0_flat_offset(full_shape, first_row: int) -> int:
    """Flat offset of a Shard(0) piece starting at `first_row`: that row times
    the product of the other dimensions ([VERL] spec.py `derive_placement`)."""
    inner = 1
    for d in full_shape[1:]:
        inner *= int(d)
    return int(first_row) * inner


def apply_(snap_bits, idx, val):
    """In-place scatter; raises ValueError if idx is not strictly ascending in range."""
    if not (isinstance(snap_bits, np.ndarray) and snap_bits.dtype == np.uint16
            and snap_bits.flags.c_contiguous):
        raise TypeError("snapshot must be a C-contiguous uint16 array")
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    val = _u16(val)
    if idx.size != val.size:
        raise ValueError("idx and val differ in length")
    rc = _load().oracle_apply(_ptr(snap_bits), snap_bits.size, _ptr(idx), _ptr(val), idx.size)
    if rc != 0:
        raise ValueError("oracle_apply: indices not strictly ascending or out of range")
    return snap_bits


def xor_mask(old_bits, new_bits):
    old_bits, new_bits = _u16(old_bits), _u16(new_bits)
    if old_bits.shape != new_bits.shape:
        raise ValueError("old and new differ in size")
    mask = np.empty_like(old_bits)
    _load().oracle_xor_mask(_ptr(old_bits), _ptr(new_bits), _ptr(mask), old_bits.size)
    return mask


def xor_apply_(snap_bits, mask):
    if not (isinstance(snap_bits, np.ndarray) and snap_bits.dtype == np.uint16
            and snap_bits.flags.c_contiguous):
        raise TypeError("snapshot must be a C-contiguous uint16 array")
    mask = _u16(mask)
    if mask.size != snap_bits.size:
        raise ValueError("mask and snapshot differ in size")
    _load().oracle_xor_apply(_ptr(snap_bits), _ptr(mask), snap_bits.size)
    return snap_bits


def bf16_rne(x: float) -> int:
    """Bit pattern of the bf16 nearest to x (ties to even)."""
    return int(_load().oracle_bf16_rne(float(x)))


def bf16_rne_array(x) -> np.ndarray:
    """Vector form of bf16_rne over a float64 array."""
    x = np.ascontiguousarray(x, dtype=np.float64).reshape(-1)
    out = np.empty(x.size, dtype=np.uint16)
    _load().oracle_bf16_rne_array(_ptr(x), _ptr(out), x.size)
    return out


def sparsity(changed: int, total: int) -> float:
    return float(_load().oracle_sparsity(int(changed), int(total)))


def touched_lines(idx, line_bytes=128, base_byte_offset=0) -> int:
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    return int(_load().oracle_touched_lines(_ptr(idx), idx.size, int(line_bytes),
                                            int(base_byte_offset)))


def wire_width(numel: int) -> int:
    return int(_load().oracle_wire_width(int(numel)))


def wire_encode(idx, offsets, numels):
    """Positions byte block of a batched delta: (positions uint8, pos_offsets int64[P+1])."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int64)
    numels = np.ascontiguousarray(numels, dtype=np.int64)
    k = numels.size
    if offsets.size != k + 1:
        raise ValueError("offsets must have nparams + 1 entries")
    positions = np.empty(max(4 * idx.size, 1), dtype=np.uint8)
    pos_offsets = np.zeros(k + 1, dtype=np.int64)
    m = _load().oracle_wire_encode(k, _ptr(numels), _ptr(idx), _ptr(offsets), _ptr(positions),
                                   _ptr(pos_offsets))
    if m < 0:
        raise ValueError("oracle_wire_encode rejected its arguments")
    return positions[:m].copy(), pos_offsets


def wire_decode(positions, pos_offsets, offsets, numels):
    positions = np.ascontiguousarray(positions, dtype=np.uint8)
    pos_offsets = np.ascontiguousarray(pos_offsets, dtype=np.int64)
    offsets = np.ascontiguousarray(offsets, dtype=np.int64)
    numels = np.ascontiguousarray(numels, dtype=np.int64)
    idx = np.empty(max(int(offsets[-1]), 1), dtype=np.int32)
    _load().oracle_wire_decode(numels.size, _ptr(numels), _ptr(positions), _ptr(pos_offsets),
                               _ptr(offsets), _ptr(idx))
    return idx[:int(offsets[-1])].copy()


def hash_bytes(b) -> int:
    b = np.ascontiguousarray(b, dtype=np.uint8)
    return int(_load().oracle_hash_bytes(_ptr(b), b.size))


def hash_bf16(bits) -> int:
    bits = _u16(bits)
    return int(_load().oracle_hash_bf16(_ptr(bits), bits.size))


def wire_checksum(positions, values_bits) -> int:
    """The flush checksum as the pages define it, on unbounded integers."""
    return hash_bytes(positions) ^ (hash_bf16(values_bits) << 1)


def wire_blocked_size(numels, entries: int) -> int:
    """Bytes of the blocked positions of `entries` entries over the list."""
    nums = np.ascontiguousarray(numels, dtype=np.int64)
    return int(_load().oracle_wire_blocked_size(nums.size, _ptr(nums), int(entries)))


def wire_encode_blocked(idx, offsets, numels) -> np.ndarray:
    """Blocked positions (uint8 bytes: the block tables, then 2-byte offsets)
    of a diff_many-layout delta."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int64)
    nums = np.ascontiguousarray(numels, dtype=np.int64)
    size = wire_blocked_size(nums, int(offsets[-1] - offsets[0]))
    out = np.zeros(max(size, 1), dtype=np.uint8)
    got = _load().oracle_wire_encode_blocked(nums.size, _ptr(nums), _ptr(idx), _ptr(offsets),
                                             _ptr(out))
    if got < 0:
        raise ValueError("oracle_wire_encode_blocked rejected the delta")
    return out[:got].copy()


def wire_decode_blocked(data, offsets, numels) -> np.ndarray:
    """int32 parameter-local indices back from blocked positions."""
    data = np.ascontiguousarray(data, dtype=np.uint8)
    offsets = np.ascontiguousarray(offsets, dtype=np.int64)
    nums = np.ascontiguousarray(numels, dtype=np.int64)
    idx = np.zeros(max(int(offsets[-1]), 1), dtype=np.int32)
    rc = _load().oracle_wire_decode_blocked(nums.size, _ptr(nums), _ptr(data), data.size,
                                            _ptr(offsets), _ptr(idx))
    if rc != 0:
        raise ValueError("oracle_wire_decode_blocked rejected the bytes")
    return idx[:int(offsets[-1])]
