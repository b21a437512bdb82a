"""torch-facing wrappers over libsbd's C ABI: argument checks and marshalling.

Every step of the hot path runs in libsbd's HIP kernels; torch supplies device
memory and the current stream only.  Names mirror the sources' callables:

  diff(old, new)                  -- per-tensor sparse delta (verl review,
                                     `shard_delta_indices`)
  diff_many(olds, news)           -- batched over a parameter list
                                     (verl review, `gather_v_batched_to_rank0`)
  apply_(snap, idx, val)          -- in-place scatter (TRL article, section 4.3)
  apply_many_(snaps, idx, val, offsets)
  xor_mask(old, new)              -- XOR-mask mode (humans& summary)
  xor_apply_(snap, mask)
  apply_streamed_(snaps, ...)     -- receiver: apply a host-resident delta
  xor_apply_streamed_(snap, mask) -- chunk by chunk, copies overlapping applies
  apply_many_host_(snaps, ...)    -- receiver: the apply kernel reads a pinned
                                     host delta itself (no staging)
  wire_encode / wire_decode / wire_checksum -- the flush's positions block
                                     and checksum (verl review, encode.py)
  wire_encode_blocked / wire_decode_blocked -- 2-byte positions for any
                                     parameter size (per-block bases)

Bit patterns travel as bfloat16 tensors (int16/uint16 views are accepted too);
indices are int32, counts and offsets int64, all on the same device.
"""
from __future__ import annotations

import ctypes
import functools
from typing import Sequence

import torch

from ._abi import DeltaError, DeltaRangeError, HostChunk, check, load

INT32_MAX = (1 << 31) - 1
_BIT_DTYPES = (torch.bfloat16, torch.int16, torch.uint16)

_workspaces: dict = {}


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _device_of(args):
    """The device of the first GPU tensor among `args` (or in a list there)."""
    for a in args:
        if isinstance(a, (list, tuple)) and a:
            a = a[0]
        if isinstance(a, torch.Tensor) and a.device.type == "cuda":
            return a.device
    return None


def _on_device(fn):
    """Run `fn` with the device of its GPU tensors current: libsbd works on the
    calling thread's current device (its streams, buffers and per-device
    state), whichever device the caller has made current."""
    @functools.wraps(fn)
    def run(*args, **kwargs):
        dev = _device_of(list(args) + list(kwargs.values()))
        if dev is None:
            return fn(*args, **kwargs)
        with torch.cuda.device(dev):
            return fn(*args, **kwargs)
    return run


def _bits(t, what: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in _BIT_DTYPES:
        # cf. the verl review: an unsupported element size is a ValueError
        raise ValueError(f"{what}: unsupported dtype {t.dtype}; expected bfloat16 bits")
    if t.device.type != "cuda":
        raise ValueError(f"{what}: must be on a GPU, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    return t


def _range(n: int, what: str):
    if n > INT32_MAX:
        raise DeltaRangeError(2, f"{what}: {n} elements exceed the int32 index range")


def workspace_size(total_elems: int, nparams: int) -> int:
    return int(load().delta_workspace_size(int(total_elems), int(nparams)))


def workspace(nbytes: int, device: torch.device) -> torch.Tensor:
    """A cached uint8 workspace per (device, stream), grown on demand.  Calls
    sharing a stream are ordered, so they may share it; release_workspaces()
    drops the cache."""
    device = torch.device(device)
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        _workspaces.pop(key, None)  # the old buffer goes back to torch first
        ws = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def release_workspaces() -> None:
    """Drop every cached workspace (after the streams that used them have
    passed their calls, e.g. after a synchronize)."""
    _workspaces.clear()


def diff_workspace_size(total_elems: int, nparams: int, capacity: int) -> int:
    """The diff's workspace for a delta of at most `capacity` entries."""
    return int(load().delta_workspace_size_for(int(total_elems), int(nparams), int(capacity)))


def default_capacity(n: int) -> int:
    """Every element when that is at most 256 MB of output, else an eighth of
    the elements plus slack; an overflow is detected and redone exactly."""
    if 6 * n <= (256 << 20):
        return n
    return n // 8 + 65536


@_on_device
def diff(old: torch.Tensor, new: torch.Tensor, capacity: int | None = None):
    """(idx int32[k], val bfloat16[k]) of the positions whose bits differ."""
    _bits(old, "old")
    _bits(new, "new")
    if old.numel() != new.numel() or old.device != new.device:
        raise ValueError("old and new must have the same numel and device")
    n = old.numel()
    _range(n, "diff")
    dev = old.device
    lib = load()
    cap = default_capacity(n) if capacity is None else int(capacity)
    nnz = torch.empty(1, dtype=torch.int64, device=dev)
    while True:
        ws = workspace(lib.delta_workspace_size_for(n, 1, cap), dev)
        idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
        val = torch.empty(max(cap, 1), dtype=torch.bfloat16, device=dev)
        check(lib.delta_diff(_ptr(old), _ptr(new), n, _ptr(idx), _ptr(val), cap, _ptr(nnz),
                             _ptr(ws), ws.numel(), _stream(dev)))
        k = int(nnz.item())  # the one device->host read
        if k <= cap:
            return idx[:k], val[:k]
        cap = k


@_on_device
def diff_many(olds: Sequence[torch.Tensor], news: Sequence[torch.Tensor],
              capacity: int | None = None, flat_offsets: Sequence[int] | None = None):
    """Batched diff: (idx_cat, val_cat bf16, nnz int64[P], offsets int64[P+1]),
    concatenated in list order.  idx_cat holds int32 parameter-local indices,
    or, when flat_offsets is given (each parameter is a rank's shard of a
    larger one), int64 global positions flat_offsets[p] + local index."""
    if len(olds) != len(news):
        raise ValueError("olds and news differ in length")
    if not olds:
        raise ValueError("empty parameter list")
    if flat_offsets is not None:
        if len(flat_offsets) != len(olds):
            raise ValueError("flat_offsets and the parameter list differ in length")
        if any(int(f) < 0 for f in flat_offsets):
            raise ValueError("flat offsets must be >= 0")
    dev = olds[0].device
    numels = []
    for p, (o, x) in enumerate(zip(olds, news)):
        _bits(o, f"olds[{p}]")
        _bits(x, f"news[{p}]")
        if o.numel() != x.numel() or o.device != dev or x.device != dev:
            raise ValueError(f"parameter {p}: numel or device mismatch")
        _range(o.numel(), f"parameter {p}")
        numels.append(o.numel())
    k = len(olds)
    total = sum(numels)
    lib = load()
    cap = default_capacity(total) if capacity is None else int(capacity)
    optrs = (ctypes.c_void_p * k)(*[o.data_ptr() for o in olds])
    nptrs = (ctypes.c_void_p * k)(*[x.data_ptr() for x in news])
    nums = (ctypes.c_int64 * k)(*numels)
    nnz = torch.empty(k, dtype=torch.int64, device=dev)
    offsets = torch.empty(k + 1, dtype=torch.int64, device=dev)
    fos = None if flat_offsets is None else (ctypes.c_int64 * k)(*[int(f) for f in flat_offsets])
    idx_dtype = torch.int32 if fos is None else torch.int64
    while True:
        ws = workspace(lib.delta_workspace_size_for(total, k, cap), dev)
        idx = torch.empty(max(cap, 1), dtype=idx_dtype, device=dev)
        val = torch.empty(max(cap, 1), dtype=torch.bfloat16, device=dev)
        if fos is None:
            check(lib.delta_diff_many(k, optrs, nptrs, nums, _ptr(idx), _ptr(val), cap,
                                      _ptr(nnz), _ptr(offsets), _ptr(ws), ws.numel(),
                                      _stream(dev)))
        else:
            check(lib.delta_diff_many_sharded(k, optrs, nptrs, nums, fos, _ptr(idx), _ptr(val),
                                              cap, _ptr(nnz), _ptr(offsets), _ptr(ws),
                                              ws.numel(), _stream(dev)))
        t = int(offsets[k].item())  # the one device->host read
        if t <= cap:
            return idx[:t], val[:t], nnz, offsets
        cap = t


def _violations(dev, enabled: bool):
    return torch.empty(1, dtype=torch.int64, device=dev) if enabled else None


def _raise_on_violations(v):
    if v is not None:
        bad = int(v.item())
        if bad:
            raise DeltaError(1, f"{bad} delta entries out of range or not strictly ascending")


@_on_device
def apply_(snap: torch.Tensor, idx: torch.Tensor, val: torch.Tensor, check_indices=False):
    """snap.view(-1)[idx] = val in place; returns snap."""
    _bits(snap, "snapshot")
    _bits(val, "val")
    if idx.dtype != torch.int32 or idx.device != snap.device or not idx.is_contiguous():
        raise ValueError("idx must be a contiguous int32 tensor on the snapshot's device")
    if idx.numel() != val.numel() or val.device != snap.device:
        raise ValueError("idx and val must have equal length on the snapshot's device")
    n = snap.numel()
    _range(n, "apply")
    lib = load()
    if check_indices:
        v = _violations(snap.device, True)
        check(lib.delta_apply_checked(_ptr(snap), n, _ptr(idx), _ptr(val), idx.numel(), _ptr(v),
                                      _stream(snap.device)))
        _raise_on_violations(v)
    else:
        check(lib.delta_apply(_ptr(snap), n, _ptr(idx), _ptr(val), idx.numel(),
                              _stream(snap.device)))
    return snap


@_on_device
def apply_many_(snaps: Sequence[torch.Tensor], idx: torch.Tensor, val: torch.Tensor,
                offsets: torch.Tensor, max_nnz: int | None = None, check_indices=False):
    """Batched in-place scatter of a diff_many result into `snaps`."""
    if not snaps:
        raise ValueError("empty parameter list")
    dev = snaps[0].device
    for p, s in enumerate(snaps):
        _bits(s, f"snaps[{p}]")
        if s.device != dev:
            raise ValueError(f"snaps[{p}] on another device")
        _range(s.numel(), f"parameter {p}")
    _bits(val, "val")
    k = len(snaps)
    if idx.dtype != torch.int32 or not idx.is_contiguous() or idx.device != dev:
        raise ValueError("idx must be a contiguous int32 tensor on the snapshots' device")
    if offsets.dtype != torch.int64 or offsets.numel() != k + 1 or offsets.device != dev:
        raise ValueError("offsets must be int64[nparams+1] on the snapshots' device")
    if val.numel() != idx.numel() or val.device != dev:
        raise ValueError("idx and val must have equal length")
    m = idx.numel() if max_nnz is None else min(int(max_nnz), idx.numel())
    lib = load()
    ws = workspace(lib.delta_workspace_size(0, k), dev)
    sptrs = (ctypes.c_void_p * k)(*[s.data_ptr() for s in snaps])
    nums = (ctypes.c_int64 * k)(*[s.numel() for s in snaps])
    v = _violations(dev, check_indices)
    check(lib.delta_apply_many(k, sptrs, nums, _ptr(idx), _ptr(val), _ptr(offsets.contiguous()),
                               m, _ptr(v) if v is not None else None, _ptr(ws), ws.numel(),
                               _stream(dev)))
    _raise_on_violations(v)
    return snaps


_stream_pairs: dict = {}


def _receiver_streams(dev: torch.device):
    """Two streams of the default priority for the streamed receiver (one for
    copies, one for applies), made once per device."""
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    if key not in _stream_pairs:
        _stream_pairs[key] = (torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev))
    return _stream_pairs[key]


def _host_bits(t, what: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or t.device.type != "cpu" or not t.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous host tensor")
    if t.dtype not in _BIT_DTYPES:
        raise ValueError(f"{what}: unsupported dtype {t.dtype}; expected bfloat16 bits")
    return t


@_on_device
def apply_many_host_(snaps: Sequence[torch.Tensor], idx: torch.Tensor, val: torch.Tensor,
                     offsets: torch.Tensor, max_nnz: int | None = None, check_indices=False,
                     wait=True):
    """apply_many_ with the delta -- idx int32, val bf16 bits, offsets
    int64[P+1], as diff_many writes them -- in host memory: idx and val must
    be pinned (pin_memory()), and the apply kernel reads them directly over
    the host link, with no device copy of the delta.  With wait=True (the
    default) the call returns once the snapshots are updated; with
    wait=False it only enqueues, and idx and val must then stay alive and
    unchanged until the current stream has passed the apply."""
    if not snaps:
        raise ValueError("empty parameter list")
    dev = snaps[0].device
    for p, s in enumerate(snaps):
        _bits(s, f"snaps[{p}]")
        if s.device != dev:
            raise ValueError(f"snaps[{p}] on another device")
        _range(s.numel(), f"parameter {p}")
    k = len(snaps)
    if (not isinstance(idx, torch.Tensor) or idx.device.type != "cpu" or idx.dtype != torch.int32
            or not idx.is_contiguous()):
        raise ValueError("idx must be a contiguous host int32 tensor")
    _host_bits(val, "val")
    if idx.numel() != val.numel():
        raise ValueError("idx and val must have equal length")
    if not (idx.numel() == 0 or (idx.is_pinned() and val.is_pinned())):
        raise ValueError("idx and val must be pinned host memory (tensor.pin_memory())")
    if (not isinstance(offsets, torch.Tensor) or offsets.device.type != "cpu" or
            offsets.dtype != torch.int64 or offsets.numel() != k + 1 or not offsets.is_contiguous()):
        raise ValueError("offsets must be a contiguous host int64 tensor of nparams + 1 entries")
    cap = idx.numel() if max_nnz is None else min(int(max_nnz), idx.numel())
    lib = load()
    ws = workspace(lib.delta_workspace_size(0, k), dev)
    sptrs = (ctypes.c_void_p * k)(*[s.data_ptr() for s in snaps])
    nums = (ctypes.c_int64 * k)(*[s.numel() for s in snaps])
    v = _violations(dev, check_indices)
    check(lib.delta_apply_many_host(k, sptrs, nums, _ptr(idx), _ptr(val), _ptr(offsets), cap,
                                    _ptr(v) if v is not None else None, _ptr(ws), ws.numel(),
                                    _stream(dev)))
    if wait or check_indices:
        torch.cuda.current_stream(dev).synchronize()
    _raise_on_violations(v)
    return snaps


@_on_device
def apply_streamed_(snaps: Sequence[torch.Tensor], idx: torch.Tensor, val: torch.Tensor,
                    offsets: torch.Tensor, bounds: Sequence[int]):
    """Apply a delta held in host memory -- idx int32, val bf16 bits, offsets
    int64[P+1], as diff_many writes them -- to the device snapshots `snaps`,
    in chunks of parameters bounds[c] .. bounds[c+1] (e.g. one layer each):
    each chunk's host-to-device copy overlaps the previous chunk's apply.
    Host tensors should be pinned.  Returns after the snapshots are updated."""
    if not snaps:
        raise ValueError("empty parameter list")
    dev = snaps[0].device
    for p, s in enumerate(snaps):
        _bits(s, f"snaps[{p}]")
        if s.device != dev:
            raise ValueError(f"snaps[{p}] on another device")
        _range(s.numel(), f"parameter {p}")
    k = len(snaps)
    if (not isinstance(idx, torch.Tensor) or idx.device.type != "cpu" or idx.dtype != torch.int32
            or not idx.is_contiguous()):
        raise ValueError("idx must be a contiguous host int32 tensor")
    _host_bits(val, "val")
    if idx.numel() != val.numel():
        raise ValueError("idx and val must have equal length")
    if (not isinstance(offsets, torch.Tensor) or offsets.device.type != "cpu" or
            offsets.dtype != torch.int64 or offsets.numel() != k + 1):
        raise ValueError("offsets must be a host int64 tensor of nparams + 1 entries")
    b = [int(x) for x in bounds]
    if not b or b[0] != 0 or b[-1] != k or any(x > y for x, y in zip(b, b[1:])):
        raise ValueError("bounds must run from 0 to nparams without decreasing")
    off = offsets.tolist()
    if off[0] != 0 or any(x > y for x, y in zip(off, off[1:])) or off[-1] > idx.numel():
        raise ValueError("offsets must start at 0, not decrease and stay within idx")
    # every chunk's offsets relative to its first entry, in one host buffer
    starts, flat = [], []
    for lo, hi in zip(b, b[1:]):
        starts.append(len(flat))
        flat.extend(x - off[lo] for x in off[lo:hi + 1])
    rel = torch.tensor(flat, dtype=torch.int64)
    chunks = (HostChunk * max(len(b) - 1, 1))()
    for c, (lo, hi) in enumerate(zip(b, b[1:])):
        chunks[c] = HostChunk(lo, hi - lo, idx.data_ptr() + 4 * off[lo],
                              val.data_ptr() + 2 * off[lo], rel.data_ptr() + 8 * starts[c])
    lib = load()
    max_p = max(hi - lo for lo, hi in zip(b, b[1:]))
    max_n = max(off[hi] - off[lo] for lo, hi in zip(b, b[1:]))
    staging = workspace(lib.delta_streamed_staging_size(k, len(b) - 1, max_p, max_n), dev)
    sptrs = (ctypes.c_void_p * k)(*[s.data_ptr() for s in snaps])
    nums = (ctypes.c_int64 * k)(*[s.numel() for s in snaps])
    cs, as_ = _receiver_streams(dev)
    # the streams start after everything already queued on the current stream
    cur = torch.cuda.current_stream(dev)
    cs.wait_stream(cur)
    as_.wait_stream(cur)
    check(lib.delta_apply_streamed(k, sptrs, nums, len(b) - 1, chunks, _ptr(staging),
                                   staging.numel(), ctypes.c_void_p(cs.cuda_stream),
                                   ctypes.c_void_p(as_.cuda_stream)))
    del rel
    return snaps


@_on_device
def xor_apply_streamed_(snap: torch.Tensor, mask: torch.Tensor, chunk_elems: int = 1 << 27):
    """snap ^= mask with `mask` in host memory (should be pinned), copied and
    applied chunk_elems elements at a time.  Returns after snap is updated."""
    _bits(snap, "snapshot")
    _host_bits(mask, "mask")
    if mask.numel() != snap.numel():
        raise ValueError("snapshot and mask must have the same numel")
    if chunk_elems <= 0:
        raise ValueError("chunk_elems must be positive")
    dev = snap.device
    lib = load()
    staging = workspace(lib.xor_streamed_staging_size(int(chunk_elems)), dev)
    cs, as_ = _receiver_streams(dev)
    cur = torch.cuda.current_stream(dev)
    cs.wait_stream(cur)
    as_.wait_stream(cur)
    check(lib.xor_apply_streamed(_ptr(snap), ctypes.c_void_p(mask.data_ptr()), snap.numel(),
                                 int(chunk_elems), _ptr(staging), staging.numel(),
                                 ctypes.c_void_p(cs.cuda_stream),
                                 ctypes.c_void_p(as_.cuda_stream)))
    return snap


def _wire_args(idx, offsets, numels):
    k = len(numels)
    if (idx.dtype != torch.int32 or not idx.is_contiguous() or idx.device.type != "cuda"
            or offsets.dtype != torch.int64 or offsets.numel() != k + 1
            or offsets.device != idx.device):
        raise ValueError("idx must be contiguous int32 on a GPU and offsets int64[nparams+1] "
                         "on the same device")
    return k, (ctypes.c_int64 * max(k, 1))(*[int(n) for n in numels])


@_on_device
def wire_encode(idx: torch.Tensor, offsets: torch.Tensor, numels: Sequence[int]):
    """Positions byte block of a diff_many result: (positions uint8, pos_offsets
    int64[P+1]) on the device; one device-to-host read of the offsets sizes it."""
    k, nums = _wire_args(idx, offsets, numels)
    dev = idx.device
    off_h = offsets.cpu().contiguous()
    size = int(load().delta_wire_positions_size(k, nums, ctypes.c_void_p(off_h.data_ptr())))
    if size < 0:
        raise ValueError("offsets or numels out of range")
    positions = torch.empty(max(size, 1), dtype=torch.uint8, device=dev)
    pos_offsets = torch.empty(k + 1, dtype=torch.int64, device=dev)
    lib = load()
    ws = workspace(lib.delta_workspace_size(0, k), dev)
    check(lib.delta_wire_encode(k, nums, _ptr(idx), _ptr(offsets),
                                min(int(off_h[-1]), idx.numel()), _ptr(positions), size,
                                _ptr(pos_offsets), _ptr(ws), ws.numel(), _stream(dev)))
    return positions[:size], pos_offsets


def _raise_on_wire_violations(v):
    bad = int(v.item())
    if bad:
        raise DeltaError(1, f"{bad} malformed entries or spans in the received positions")


@_on_device
def wire_decode(positions: torch.Tensor, pos_offsets: torch.Tensor, offsets: torch.Tensor,
                numels: Sequence[int]) -> torch.Tensor:
    """int32 parameter-local indices back from a positions block (which may
    come from a remote sender: the library reads nothing outside it and
    counts malformed entries, which raise here)."""
    k = len(numels)
    dev = positions.device
    if (positions.dtype != torch.uint8 or not positions.is_contiguous() or dev.type != "cuda"
            or pos_offsets.dtype != torch.int64 or pos_offsets.numel() != k + 1
            or pos_offsets.device != dev or offsets.dtype != torch.int64
            or offsets.numel() != k + 1 or offsets.device != dev):
        raise ValueError("positions must be contiguous uint8 on a GPU, pos_offsets and offsets "
                         "int64[nparams+1] on the same device")
    total = int(offsets[k].item())
    if total < 0:
        raise ValueError("offsets give a negative entry count")
    idx = torch.empty(max(total, 1), dtype=torch.int32, device=dev)
    v = torch.empty(1, dtype=torch.int64, device=dev)
    lib = load()
    ws = workspace(lib.delta_workspace_size(0, k), dev)
    nums = (ctypes.c_int64 * max(k, 1))(*[int(n) for n in numels])
    check(lib.delta_wire_decode(k, nums, _ptr(positions), positions.numel(), _ptr(pos_offsets),
                                _ptr(offsets), total, _ptr(idx), _ptr(v), _ptr(ws), ws.numel(),
                                _stream(dev)))
    _raise_on_wire_violations(v)
    return idx[:total]


@_on_device
def wire_encode_blocked(idx: torch.Tensor, offsets: torch.Tensor, numels: Sequence[int]):
    """Blocked positions (2 bytes per position for any parameter size) of a
    diff_many result, as a uint8 device tensor; one device-to-host read of
    the total sizes it."""
    k, nums = _wire_args(idx, offsets, numels)
    dev = idx.device
    total = min(int(offsets[k].item()), idx.numel())
    lib = load()
    size = int(lib.delta_wire_blocked_size(k, nums, total))
    if size < 0:
        raise ValueError("numels out of range")
    out = torch.empty(max(size, 1), dtype=torch.uint8, device=dev)
    ws = workspace(lib.delta_workspace_size(0, k), dev)
    check(lib.delta_wire_encode_blocked(k, nums, _ptr(idx), _ptr(offsets), total, _ptr(out), size,
                                        _ptr(ws), ws.numel(), _stream(dev)))
    return out[:size]


@_on_device
def wire_decode_blocked(data: torch.Tensor, offsets: torch.Tensor,
                        numels: Sequence[int]) -> torch.Tensor:
    """int32 parameter-local indices back from blocked positions (untrusted
    bytes: nothing outside them is read; malformed entries raise)."""
    k = len(numels)
    dev = data.device
    if (data.dtype != torch.uint8 or not data.is_contiguous() or dev.type != "cuda"
            or offsets.dtype != torch.int64 or offsets.numel() != k + 1 or offsets.device != dev):
        raise ValueError("data must be contiguous uint8 on a GPU and offsets int64[nparams+1] "
                         "on the same device")
    total = int(offsets[k].item())
    if total < 0:
        raise ValueError("offsets give a negative entry count")
    idx = torch.empty(max(total, 1), dtype=torch.int32, device=dev)
    v = torch.empty(1, dtype=torch.int64, device=dev)
    lib = load()
    ws = workspace(lib.delta_workspace_size(0, k), dev)
    nums = (ctypes.c_int64 * max(k, 1))(*[int(n) for n in numels])
    check(lib.delta_wire_decode_blocked(k, nums, _ptr(data), data.numel(), _ptr(offsets), total,
                                        _ptr(idx), _ptr(v), _ptr(ws), ws.numel(), _stream(dev)))
    _raise_on_wire_violations(v)
    return idx[:total]


@_on_device
def wire_hashes(positions: torch.Tensor, values: torch.Tensor) -> tuple[int, int]:
    """(hash of the position bytes, hash of the bf16 values) as unsigned ints."""
    _bits(values, "values")
    if positions.dtype != torch.uint8 or positions.device != values.device:
        raise ValueError("positions must be uint8 on the values' device")
    h = torch.empty(2, dtype=torch.int64, device=values.device)
    check(load().delta_wire_hash(_ptr(positions), positions.numel(), _ptr(values),
                                 values.numel(), _ptr(h), _stream(values.device)))
    a, b = h.cpu().tolist()
    return a & (2 ** 64 - 1), b & (2 ** 64 - 1)


@_on_device
def wire_checksum(positions: torch.Tensor, values: torch.Tensor) -> int:
    """The flush checksum hash(positions) ^ (hash(values) << 1), computed by
    the library as 65 bits in two words, returned as one Python int."""
    _bits(values, "values")
    if positions.dtype != torch.uint8 or positions.device != values.device:
        raise ValueError("positions must be uint8 on the values' device")
    c = torch.empty(2, dtype=torch.int64, device=values.device)
    check(load().delta_wire_checksum(_ptr(positions), positions.numel(), _ptr(values),
                                     values.numel(), _ptr(c), _stream(values.device)))
    lo, hi = (x & (2 ** 64 - 1) for x in c.cpu().tolist())
    return lo | (hi << 64)


@_on_device
def xor_mask(old: torch.Tensor, new: torch.Tensor, out: torch.Tensor | None = None):
    """mask = old ^ new (bit patterns) as an int16 tensor shaped like old."""
    _bits(old, "old")
    _bits(new, "new")
    if old.numel() != new.numel() or old.device != new.device:
        raise ValueError("old and new must have the same numel and device")
    if out is None:
        out = torch.empty(old.shape, dtype=torch.int16, device=old.device)
    else:
        _bits(out, "out")
        if out.numel() != old.numel() or out.device != old.device:
            raise ValueError("out must match old in numel and device")
    check(load().xor_mask(_ptr(old), _ptr(new), _ptr(out), old.numel(), _stream(old.device)))
    return out


@_on_device
def xor_apply_(snap: torch.Tensor, mask: torch.Tensor):
    """snap ^= mask in place; returns snap."""
    _bits(snap, "snapshot")
    _bits(mask, "mask")
    if snap.numel() != mask.numel() or snap.device != mask.device:
        raise ValueError("snapshot and mask must have the same numel and device")
    check(load().xor_apply(_ptr(snap), _ptr(mask), snap.numel(), _stream(snap.device)))
    return snap
