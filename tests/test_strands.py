"""The two-strand pairing: the exhaustive reference (oracle/strands.py) pinned by closed forms and a
worked example, and the library's dynamic program (tpslice_strand_schedule) against it on random
profiles (the check that the micro-batch co-execution review proposes under "What would settle it":
the recurrence's plan against exhaustive search)."""
import ctypes
import math
import random

import pytest

from oracle import strands as S

T = pytest.importorskip("comm_overlap_amd.tpslice", reason="libtpslice.so not built")


def delannoy(m, n):
    """Monotone lattice paths with right, down and diagonal steps: sum_k C(m, k) C(n, k) 2^k."""
    return sum(math.comb(m, k) * math.comb(n, k) * 2 ** k for k in range(min(m, n) + 1))


@pytest.mark.parametrize("nf,nb", [(0, 0), (1, 0), (0, 3), (1, 1), (2, 2), (3, 2), (4, 4), (5, 3)])
def test_every_pairing_is_enumerated_once(nf, nb):
    ps = S.pairings(nf, nb)
    assert len(ps) == delannoy(nf, nb)
    assert len({tuple(p) for p in ps}) == len(ps)
    for p in ps:
        assert [i for i, _ in p if i] == list(range(1, nf + 1))
        assert [j for _, j in p if j] == list(range(1, nb + 1))


# A worked example (two forward, two backward segments), solved by hand: solos F1 = 3, F2 = 2,
# B1 = 4, B2 = 1; pairs (1,1) = 5, (1,2) = 3.5, (2,1) = 4.5, (2,2) = 2.5. Pairing F1 with B1 and F2
# with B2 costs 5 + 2.5 = 7.5; every other pairing costs more: F1 with B1 then the rest alone 8,
# F1 alone, F2 with B1, B2 alone 8.5, B1 alone, F1 with B2, F2 alone 9.5, all alone 10.
EXAMPLE = [[0.0, 4.0, 1.0], [3.0, 5.0, 3.5], [2.0, 4.5, 2.5]]


def test_worked_example():
    m, opt = S.best(EXAMPLE)
    assert m == 7.5 and opt == [[(1, 1), (2, 2)]]
    assert S.cost(EXAMPLE, [(1, 1), (2, 0), (0, 2)]) == 8.0
    assert S.cost(EXAMPLE, [(1, 0), (2, 0), (0, 1), (0, 2)]) == 10.0
    steps, t = T.strand_schedule(EXAMPLE)
    assert steps == [(1, 1), (2, 2)] and t == 7.5


def test_pairs_that_save_nothing():
    """A pair costing exactly its two solos: every pairing costs the sum of all solos."""
    rng = random.Random(3)
    f = [rng.uniform(1, 5) for _ in range(3)]
    b = [rng.uniform(1, 5) for _ in range(4)]
    P = [[0.0] + b] + [[fi] + [fi + bj for bj in b] for fi in f]
    m, opt = S.best(P)
    assert m == pytest.approx(sum(f) + sum(b), rel=1e-12)
    assert len(opt) >= 1
    _, t = T.strand_schedule(P)
    assert t == pytest.approx(m, rel=1e-12)


def test_free_pairs_on_equal_strands():
    """Pairs costing the longer of their two segments, with equal per-step segments: the diagonal
    pairing (every step a pair) is optimal and costs the sum of the longer ones."""
    f = [3.0, 1.0, 2.0]
    b = [2.0, 2.0, 2.0]
    P = [[0.0] + b] + [[fi] + [max(fi, bj) for bj in b] for fi in f]
    m, opt = S.best(P)
    assert m == sum(max(x, y) for x, y in zip(f, b))
    assert [(1, 1), (2, 2), (3, 3)] in opt


@pytest.mark.parametrize("seed", range(40))
def test_dynamic_program_matches_exhaustive_search(seed):
    rng = random.Random(seed)
    nf, nb = rng.randint(0, 5), rng.randint(0, 5)
    integer = seed % 2 == 0  # integer times: ties are exact, so the optimum is compared exactly
    draw = (lambda: float(rng.randint(1, 9))) if integer else (lambda: rng.uniform(0.5, 3.0))
    P = [[0.0] * (nb + 1) for _ in range(nf + 1)]
    for i in range(nf + 1):
        for j in range(nb + 1):
            if i or j:
                P[i][j] = draw()
    for i in range(1, nf + 1):  # pairs between the longer solo and the sum of both, as on a GPU
        for j in range(1, nb + 1):
            lo, hi = max(P[i][0], P[0][j]), P[i][0] + P[0][j]
            P[i][j] = float(rng.randint(int(lo), int(hi))) if integer else rng.uniform(lo, hi)
    m, opt = S.best(P)
    steps, t = T.strand_schedule(P)
    if integer:
        assert t == m
    else:
        assert t == pytest.approx(m, rel=1e-12)
    assert S.cost(P, steps) == pytest.approx(t, rel=1e-12)
    if integer:
        assert steps in opt
    assert [i for i, _ in steps if i] == list(range(1, nf + 1))
    assert [j for _, j in steps if j] == list(range(1, nb + 1))


def test_schedule_argument_errors():
    lib = T.lib
    P = (ctypes.c_double * 9)(*[0.0] + [1.0] * 8)
    steps = (ctypes.c_int32 * 8)()
    n, t = ctypes.c_int32(), ctypes.c_double()
    assert lib.tpslice_strand_schedule(None, 2, 2, steps, ctypes.byref(n), ctypes.byref(t)) == T.ERR_INVALID
    assert lib.tpslice_strand_schedule(P, -1, 2, steps, ctypes.byref(n), ctypes.byref(t)) == T.ERR_SHAPE
    assert lib.tpslice_strand_schedule(P, 5000, 0, steps, ctypes.byref(n), ctypes.byref(t)) == T.ERR_SHAPE
    bad = (ctypes.c_double * 9)(*[0.0, 1.0, 1.0, 1.0, -2.0, 1.0, 1.0, 1.0, 1.0])
    assert lib.tpslice_strand_schedule(bad, 2, 2, steps, ctypes.byref(n), ctypes.byref(t)) == T.ERR_INVALID
    nan = (ctypes.c_double * 9)(*[0.0, 1.0, 1.0, 1.0, float("nan"), 1.0, 1.0, 1.0, 1.0])
    assert lib.tpslice_strand_schedule(nan, 2, 2, steps, ctypes.byref(n), ctypes.byref(t)) == T.ERR_INVALID
    assert lib.tpslice_strand_schedule(P, 0, 0, steps, ctypes.byref(n), ctypes.byref(t)) == T.OK
    assert n.value == 0 and t.value == 0.0
