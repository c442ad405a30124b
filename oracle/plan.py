"""Slice geometry of the sliced layer shard: which rows and columns each independent piece owns.

TEST INFRASTRUCTURE (see oracle/layer.py). Integer work, checked bit-exactly against the library's
planner.

Domino page, Abstract: one batch's work is broken into smaller independent pieces whose hand-off is
overlapped with later pieces' compute. The pieces here are contiguous, equal token-row ranges of the
batch (row slices), each further cut into equal column ranges of the partial-sum output (column
slices), so every piece of the hand-off tensor is finished by its own product. The plainest reading
of "independent pieces": equal contiguous ranges, in ascending order, row slice major.
"""
from __future__ import annotations

from typing import List, Tuple


def even_ranges(n: int, parts: int) -> List[Tuple[int, int]]:
    """[(begin, end)) of `parts` equal contiguous ranges covering [0, n). Requires parts | n."""
    if parts <= 0 or n <= 0 or n % parts:
        raise ValueError(f"{parts} equal parts do not tile {n}")
    step = n // parts
    return [(p * step, (p + 1) * step) for p in range(parts)]


def handoff_pieces(rows: int, cols: int, r: int, c: int) -> List[Tuple[int, int, int, int]]:
    """Pieces (row_begin, row_end, col_begin, col_end) of a [rows][cols] hand-off tensor in the
    order they are finished: row slice i ascending, then column slice j ascending."""
    out = []
    for (r0, r1) in even_ranges(rows, r):
        for (c0, c1) in even_ranges(cols, c):
            out.append((r0, r1, c0, c1))
    return out
