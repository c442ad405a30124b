"""Plain CPU reference of the two-strand pairing (TEST INFRASTRUCTURE: only the test suite and the
benchmark may import it; the product path never does, and it shares no code with the library).

The forward segments 1..nf of one micro-batch and the backward segments 1..nb of another run in
order within each strand. A pairing is a sequence of steps, each running one forward segment alone,
one backward segment alone, or one of each side by side, that uses every segment once in order
(a monotone path from (0, 0) to (nf, nb) with unit right, down and diagonal moves). Its makespan is
the sum of its steps' measured times P (micro-batch co-execution review, "What carries the
argument": the planner adds up pairwise profiled times, and takes the best pairing). Here every
pairing is enumerated and costed, so the best one is found by exhaustive search, not by the
review's recurrence.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

Step = Tuple[int, int]


def pairings(nf: int, nb: int) -> List[List[Step]]:
    """Every pairing, each a list of (forward, backward) segment numbers (0 = none)."""
    out: List[List[Step]] = []

    def walk(i: int, j: int, path: List[Step]):
        if i == nf and j == nb:
            out.append(list(path))
            return
        if i < nf:
            path.append((i + 1, 0)); walk(i + 1, j, path); path.pop()
        if j < nb:
            path.append((0, j + 1)); walk(i, j + 1, path); path.pop()
        if i < nf and j < nb:
            path.append((i + 1, j + 1)); walk(i + 1, j + 1, path); path.pop()

    walk(0, 0, [])
    return out


def cost(P: Sequence[Sequence[float]], steps: Sequence[Step]) -> float:
    """Sum of the steps' times: P[i][j] for a pair, P[i][0] / P[0][j] for a segment alone."""
    return float(sum(P[i][j] for i, j in steps))


def best(P: Sequence[Sequence[float]]) -> Tuple[float, List[List[Step]]]:
    """The least makespan over all pairings and every pairing that reaches it."""
    nf, nb = len(P) - 1, len(P[0]) - 1
    costs = [(cost(P, s), s) for s in pairings(nf, nb)]
    m = min(c for c, _ in costs)
    return m, [s for c, s in costs if c == m]
