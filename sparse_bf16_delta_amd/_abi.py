"""ctypes declarations for libsbd's C ABI (include/sbd.h).

torch is imported before the library is loaded on purpose: torch's bundled
HIP runtime and ROCm's share the soname ``libamdhip64.so.7``, so loading torch
first makes libsbd bind to the very runtime that owns torch's streams and
allocations (one runtime per process).

Loading fails loudly when ``libsbd.so`` has not been built: there is no
fallback implementation of any entry point.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede the CDLL load; see module docstring)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsbd.so")

DELTA_OK = 0
DELTA_E_INVALID = 1
DELTA_E_RANGE = 2
DELTA_E_WORKSPACE = 3
DELTA_E_HIP = 4

STATUS_NAMES = {
    DELTA_OK: "DELTA_OK",
    DELTA_E_INVALID: "DELTA_E_INVALID",
    DELTA_E_RANGE: "DELTA_E_RANGE",
    DELTA_E_WORKSPACE: "DELTA_E_WORKSPACE",
    DELTA_E_HIP: "DELTA_E_HIP",
}

class HostChunk(ctypes.Structure):
    """delta_host_chunk of include/sbd.h."""
    _fields_ = [("first_param", ctypes.c_int32), ("nparams", ctypes.c_int32),
                ("idx", ctypes.c_void_p), ("val", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p)]


# name -> (restype, argtypes); mirrors include/sbd.h
_i64, _i32, _sz, _vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
_st = ctypes.c_int
SIGNATURES = {
    "delta_workspace_size": (_sz, [_i64, _i32]),
    "delta_workspace_size_for": (_sz, [_i64, _i32, _i64]),
    "delta_diff": (_st, [_vp, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _sz, _vp]),
    "delta_diff_noalloc": (_st, [_vp, _vp, _i64, _vp, _vp, _i64, _vp, _vp]),
    "delta_diff_noalloc_max_elems": (_i64, []),
    "delta_diff_many": (_st, [_i32, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "delta_diff_many_sharded": (_st, [_i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp,
                                      _sz, _vp]),
    "delta_apply": (_st, [_vp, _i64, _vp, _vp, _i64, _vp]),
    "delta_apply_checked": (_st, [_vp, _i64, _vp, _vp, _i64, _vp, _vp]),
    "delta_apply_many": (_st, [_i32, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _sz, _vp]),
    "delta_streamed_staging_size": (_sz, [_i32, _i32, _i32, _i64]),
    "delta_apply_streamed": (_st, [_i32, _vp, _vp, _i32, _vp, _vp, _sz, _vp, _vp]),
    "delta_apply_many_host": (_st, [_i32, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _sz, _vp]),
    "xor_streamed_staging_size": (_sz, [_i64]),
    "xor_apply_streamed": (_st, [_vp, _vp, _i64, _i64, _vp, _sz, _vp, _vp]),
    "delta_wire_encode": (_st, [_i32, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _vp, _sz, _vp]),
    "delta_wire_positions_size": (_i64, [_i32, _vp, _vp]),
    "delta_wire_decode": (_st, [_i32, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "delta_wire_hash": (_st, [_vp, _i64, _vp, _i64, _vp, _vp]),
    "delta_wire_checksum": (_st, [_vp, _i64, _vp, _i64, _vp, _vp]),
    "delta_wire_blocked_size": (_i64, [_i32, _vp, _i64]),
    "delta_wire_encode_blocked": (_st, [_i32, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _sz, _vp]),
    "delta_wire_decode_blocked": (_st, [_i32, _vp, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _sz,
                                        _vp]),
    "xor_mask": (_st, [_vp, _vp, _vp, _i64, _vp]),
    "xor_apply": (_st, [_vp, _vp, _i64, _vp]),
    "delta_last_error": (ctypes.c_char_p, []),
}


class DeltaError(RuntimeError):
    """A libsbd entry point returned a non-OK delta_status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class DeltaRangeError(DeltaError, OverflowError):
    pass


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libsbd.so is not built ({LIB_PATH}); run `python -m sparse_bf16_delta_amd.build` "
            "or __graft_entry__.build() -- there is no CPU fallback")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != DELTA_OK:
        msg = load().delta_last_error().decode(errors="replace")
        if status == DELTA_E_RANGE:
            raise DeltaRangeError(status, msg)
        raise DeltaError(status, msg)
