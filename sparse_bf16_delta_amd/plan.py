"""Persistent plans for a fixed parameter list: the per-step sync loop of an
RL trainer calls the C ABI with buffers allocated once, and reads nothing
back unless asked.

An RL run syncs the same parameters every step, so the pointer arrays, the
workspace and a delta buffer of fixed capacity are built once.  A step then
costs one ctypes call per side; the true count lands in device memory and is
read only when the caller needs it (TRL article section 4.2: one delta per
optimizer step; verl review notes: one stacked device-to-host read).
"""
from __future__ import annotations

import ctypes
from typing import Sequence

import torch

from ._abi import DeltaError, HostChunk, check, load
from .ops import _BIT_DTYPES, _bits, _ptr, _range, _stream


class DiffPlan:
    """Sender side: delta_diff_many over fixed (old, new) snapshot lists."""

    def __init__(self, olds: Sequence[torch.Tensor], news: Sequence[torch.Tensor],
                 capacity: int, flat_offsets: Sequence[int] | None = None):
        """flat_offsets: each parameter is a rank's shard of a larger one,
        starting at that flat offset; the delta then holds int64 global
        positions (delta_diff_many_sharded)."""
        if len(olds) != len(news) or not olds:
            raise ValueError("need two equally long, non-empty parameter lists")
        self.device = olds[0].device
        for p, (o, x) in enumerate(zip(olds, news)):
            _bits(o, f"olds[{p}]")
            _bits(x, f"news[{p}]")
            if o.numel() != x.numel() or o.device != self.device or x.device != self.device:
                raise ValueError(f"parameter {p}: numel or device mismatch")
            _range(o.numel(), f"parameter {p}")
        self.nparams = k = len(olds)
        self.numels = [o.numel() for o in olds]
        self.total = sum(self.numels)
        self.capacity = int(capacity)
        self._keep = (list(olds), list(news))
        self._optrs = (ctypes.c_void_p * k)(*[o.data_ptr() for o in olds])
        self._nptrs = (ctypes.c_void_p * k)(*[x.data_ptr() for x in news])
        self._nums = (ctypes.c_int64 * k)(*self.numels)
        lib = load()
        dev = self.device
        # the minimum plus a staging arena for `capacity` entries
        self.ws = torch.empty(lib.delta_workspace_size_for(self.total, k, self.capacity),
                              dtype=torch.uint8, device=dev)
        if flat_offsets is not None and (len(flat_offsets) != k or
                                         any(int(f) < 0 for f in flat_offsets)):
            raise ValueError("need one flat offset >= 0 per parameter")
        self._fos = None if flat_offsets is None else (ctypes.c_int64 * k)(*map(int, flat_offsets))
        self.idx = torch.empty(max(self.capacity, 1),
                               dtype=torch.int32 if self._fos is None else torch.int64, device=dev)
        self.val = torch.empty(max(self.capacity, 1), dtype=torch.bfloat16, device=dev)
        self.nnz = torch.empty(k, dtype=torch.int64, device=dev)
        self.offsets = torch.empty(k + 1, dtype=torch.int64, device=dev)

    def run(self):
        """Enqueue the diff on the current stream; returns without syncing."""
        lib = load()
        with torch.cuda.device(self.device):  # the library works on the current device
            if self._fos is None:
                check(lib.delta_diff_many(self.nparams, self._optrs, self._nptrs, self._nums,
                                          _ptr(self.idx), _ptr(self.val), self.capacity,
                                          _ptr(self.nnz), _ptr(self.offsets), _ptr(self.ws),
                                          self.ws.numel(), _stream(self.device)))
            else:
                check(lib.delta_diff_many_sharded(self.nparams, self._optrs, self._nptrs,
                                                  self._nums, self._fos, _ptr(self.idx),
                                                  _ptr(self.val), self.capacity, _ptr(self.nnz),
                                                  _ptr(self.offsets), _ptr(self.ws),
                                                  self.ws.numel(), _stream(self.device)))

    def changed(self) -> int:
        """True total count of the last run (one device-to-host read)."""
        return int(self.offsets[self.nparams].item())

    def result(self):
        """(idx, val, nnz, offsets) of the last run; raises if the capacity was
        too small (the caller re-plans with a larger one)."""
        t = self.changed()
        if t > self.capacity:
            raise DeltaError(3, f"delta of {t} entries exceeds the capacity {self.capacity}")
        return self.idx[:t], self.val[:t], self.nnz, self.offsets


class ApplyPlan:
    """Receiver side: delta_apply_many into fixed resident snapshots."""

    def __init__(self, snaps: Sequence[torch.Tensor]):
        if not snaps:
            raise ValueError("empty parameter list")
        self.device = snaps[0].device
        for p, s in enumerate(snaps):
            _bits(s, f"snaps[{p}]")
            if s.device != self.device:
                raise ValueError(f"snaps[{p}] on another device")
            _range(s.numel(), f"parameter {p}")
        self.nparams = k = len(snaps)
        self._keep = list(snaps)
        self._sptrs = (ctypes.c_void_p * k)(*[s.data_ptr() for s in snaps])
        self._nums = (ctypes.c_int64 * k)(*[s.numel() for s in snaps])
        self.ws = torch.empty(load().delta_workspace_size(0, k), dtype=torch.uint8,
                              device=self.device)

    def run(self, idx: torch.Tensor, val: torch.Tensor, offsets: torch.Tensor,
            max_nnz: int | None = None, violations: torch.Tensor | None = None):
        """Enqueue the scatter of a diff_many-layout delta; returns without syncing.
        Entries j < min(offsets[nparams], max_nnz) are applied.  Pass the true
        count as max_nnz when it is known: the kernel is chosen from it, and a
        sparse delta applied with only the buffer's capacity runs the general
        kernel (about 14 % slower on a 7B-shaped delta at 1.2 %)."""
        dev = self.device
        _bits(val, "val")
        if idx.dtype != torch.int32 or not idx.is_contiguous() or idx.device != dev:
            raise ValueError("idx must be a contiguous int32 tensor on the snapshots' device")
        if val.numel() != idx.numel() or val.device != dev:
            raise ValueError("idx and val must have equal length on the snapshots' device")
        if (offsets.numel() != self.nparams + 1 or offsets.dtype != torch.int64
                or not offsets.is_contiguous() or offsets.device != dev):
            raise ValueError("offsets must be a contiguous int64[nparams+1] on the snapshots' "
                             "device")
        if violations is not None and (violations.dtype != torch.int64 or
                                       violations.device != dev):
            raise ValueError("violations must be an int64 tensor on the snapshots' device")
        # the kernel never reads past the buffers, whatever the device offsets say
        m = idx.numel() if max_nnz is None else min(int(max_nnz), idx.numel())
        with torch.cuda.device(dev):  # the library works on the current device
            check(load().delta_apply_many(self.nparams, self._sptrs, self._nums, _ptr(idx),
                                          _ptr(val), _ptr(offsets), m,
                                          _ptr(violations) if violations is not None else None,
                                          _ptr(self.ws), self.ws.numel(), _stream(dev)))


class StreamedApplyPlan:
    """Receiver side with the delta in host memory: delta_apply_streamed over
    fixed resident snapshots and fixed chunk bounds (parameters
    bounds[c] .. bounds[c+1], e.g. groups of layers).  The snapshot table,
    staging buffer and the two streams are made once; a step builds only the
    chunk table.  A few large chunks stream best: every chunk costs two
    host-to-device copies plus a fixed overhead."""

    def __init__(self, snaps: Sequence[torch.Tensor], bounds: Sequence[int],
                 max_chunk_nnz: int):
        from .ops import _receiver_streams

        if not snaps:
            raise ValueError("empty parameter list")
        self.device = snaps[0].device
        for p, s in enumerate(snaps):
            _bits(s, f"snaps[{p}]")
            if s.device != self.device:
                raise ValueError(f"snaps[{p}] on another device")
            _range(s.numel(), f"parameter {p}")
        self.nparams = k = len(snaps)
        b = [int(x) for x in bounds]
        if not b or b[0] != 0 or b[-1] != k or any(x > y for x, y in zip(b, b[1:])):
            raise ValueError("bounds must run from 0 to nparams without decreasing")
        self.bounds = b
        self.nchunks = len(b) - 1
        self.max_chunk_nnz = int(max_chunk_nnz)
        self._keep = list(snaps)
        self._sptrs = (ctypes.c_void_p * k)(*[s.data_ptr() for s in snaps])
        self._nums = (ctypes.c_int64 * k)(*[s.numel() for s in snaps])
        max_p = max(hi - lo for lo, hi in zip(b, b[1:]))
        self.staging = torch.empty(
            load().delta_streamed_staging_size(k, self.nchunks, max_p, self.max_chunk_nnz),
            dtype=torch.uint8, device=self.device)
        self._chunks = (HostChunk * max(self.nchunks, 1))()
        self._streams = _receiver_streams(self.device)

    def run(self, idx: torch.Tensor, val: torch.Tensor, offsets: torch.Tensor):
        """Apply a host delta (int32 idx, bf16-bit val, int64 offsets[nparams+1]
        as diff_many writes them; pinned for the copies to overlap).  Returns
        after the snapshots are updated."""
        if (idx.device.type != "cpu" or val.device.type != "cpu" or offsets.device.type != "cpu"
                or idx.dtype != torch.int32 or offsets.dtype != torch.int64
                or offsets.numel() != self.nparams + 1 or not idx.is_contiguous()
                or not val.is_contiguous() or val.dtype not in _BIT_DTYPES):
            raise ValueError("idx int32, val (bf16 bits) and offsets int64[nparams+1] must be "
                             "contiguous host tensors")
        if idx.numel() != val.numel():
            raise ValueError("idx and val must have equal length")
        off = offsets.tolist()
        if off[0] != 0 or any(x > y for x, y in zip(off, off[1:])) or off[-1] > idx.numel():
            raise ValueError("offsets must start at 0, not decrease and stay within idx")
        b = self.bounds
        rel = torch.empty(self.nparams + self.nchunks, dtype=torch.int64)
        r = rel.numpy()
        pos = 0
        for c, (lo, hi) in enumerate(zip(b, b[1:])):
            if off[hi] - off[lo] > self.max_chunk_nnz:
                raise DeltaError(3, f"chunk {c} holds {off[hi] - off[lo]} entries, more than "
                                    f"the plan's {self.max_chunk_nnz}")
            r[pos:pos + hi - lo + 1] = [x - off[lo] for x in off[lo:hi + 1]]
            self._chunks[c] = HostChunk(lo, hi - lo, idx.data_ptr() + 4 * off[lo],
                                        val.data_ptr() + 2 * off[lo],
                                        rel.data_ptr() + 8 * pos)
            pos += hi - lo + 1
        cs, as_ = self._streams
        cur = torch.cuda.current_stream(self.device)
        cs.wait_stream(cur)
        as_.wait_stream(cur)
        with torch.cuda.device(self.device):  # the library works on the current device
            check(load().delta_apply_streamed(self.nparams, self._sptrs, self._nums,
                                              self.nchunks, self._chunks, _ptr(self.staging),
                                              self.staging.numel(),
                                              ctypes.c_void_p(cs.cuda_stream),
                                              ctypes.c_void_p(as_.cuda_stream)))
