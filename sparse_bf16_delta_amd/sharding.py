"""Shard(0) placement for the sharded diff (host side).

Under FSDP2 each parameter is split along its first dimension: the verl
review's spec.py `derive_placement` takes the global offset of a rank's
piece and turns it into a flat offset, first row times the product of the
other dimensions.  `delta_diff_many_sharded` adds that offset to every local
index, so the ranks' deltas of a parameter, concatenated in rank order, are
the whole parameter's delta.
"""
from __future__ import annotations

from math import prod
from typing import Sequence


def shard0_piece(rows: int, world: int, rank: int) -> tuple[int, int]:
    """(first_row, row_count) of `rank`'s piece of `rows` rows over `world`
    ranks: pieces of ceil(rows / world) rows in rank order, the last ones
    shorter or empty (the Shard(0) split)."""
    if rows < 0 or world < 1 or not 0 <= rank < world:
        raise ValueError(f"bad shard geometry rows={rows} world={world} rank={rank}")
    per_rank = -(-rows // world)
    start = min(rank * per_rank, rows)
    return start, min(per_rank, rows - start)


def flat_offset(full_shape: Sequence[int], first_row: int) -> int:
    """Flat (row-major) offset of row `first_row` of a tensor of `full_shape`."""
    if not full_shape:
        raise ValueError("a scalar has no rows to shard")
    if not 0 <= first_row <= full_shape[0]:
        raise ValueError(f"row {first_row} outside 0..{full_shape[0]}")
    return int(first_row) * prod(int(d) for d in full_shape[1:])
