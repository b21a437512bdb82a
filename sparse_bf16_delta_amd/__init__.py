"""sparse_bf16_delta_amd -- the data-parallel hot path of bf16 delta weight sync
for asynchronous RL on AMD Instinct MI355X (gfx950).

Sender: bitwise change detection between the pre-step and post-step bf16
snapshots, compacted into (ascending int32 indices, bf16 values).  Receiver:
in-place scatter of that delta into a resident snapshot.  Second mode: the
full-size XOR mask.  All of it runs in hand-written HIP kernels in
``libsbd.so`` behind the C ABI of ``include/sbd.h``; this package only
marshals torch tensors into that ABI.
"""
from ._abi import DeltaError, DeltaRangeError, load  # noqa: F401
from .ops import (  # noqa: F401
    apply_,
    apply_many_,
    apply_many_host_,
    apply_streamed_,
    default_capacity,
    diff,
    diff_workspace_size,
    release_workspaces,
    diff_many,
    workspace,
    workspace_size,
    xor_apply_,
    xor_apply_streamed_,
    xor_mask,
    wire_checksum,
    wire_decode,
    wire_decode_blocked,
    wire_encode,
    wire_encode_blocked,
    wire_hashes,
)
from .sharding import flat_offset, shard0_piece  # noqa: F401

__all__ = [
    "DeltaError", "DeltaRangeError", "load", "diff", "diff_many", "apply_", "apply_many_",
    "xor_mask", "xor_apply_", "workspace", "workspace_size", "default_capacity",
    "shard0_piece", "flat_offset", "apply_streamed_", "xor_apply_streamed_", "apply_many_host_",
    "wire_encode", "wire_decode", "wire_hashes", "wire_checksum", "wire_encode_blocked",
    "wire_decode_blocked", "diff_workspace_size", "release_workspaces",
]
