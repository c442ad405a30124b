"""Two strands paired segment by segment (comm_overlap_amd/strands.py) give the bits of the same
segments run in sequence, whatever the pairing: the pairing only reorders and overlaps calls of
independent micro-batches (micro-batch co-execution review, "If this is right": training semantics
are unchanged)."""
import pytest
import torch

from comm_overlap_amd import synth

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from comm_overlap_amd import strands as ST

SMALL = synth.custom("strands", 960, tokens=1024, hidden=512, ffn=2048, tp=2, act="swiglu", bias=False,
                     row_slices=4, col_slices=2, heads=8, kv_heads=2, head_dim=64, backward=True)


def _snapshot(sp):
    torch.cuda.synchronize()
    return {k: v.clone() for d in (sp.a, sp.b, sp.g) for k, v in d.items()}


def test_pairings_change_no_result():
    print(f"[case] strands {SMALL.key}", flush=True)
    inp = synth.make_inputs(SMALL)
    dev = {k: v.to("cuda").contiguous() for k, v in inp.items()}
    sp = ST.StrandPair(SMALL, dev)
    try:
        sp.enqueue(sp.sequential())
        ref = _snapshot(sp)
        P = sp.profile(reps=1)
        steps, predicted = ST.schedule(P)
        assert predicted > 0 and len(steps) >= len(sp.fwd)
        diag = [(k + 1, k + 1) for k in range(len(sp.fwd))]
        mixed = [(0, 1), (1, 2), (2, 0), (3, 3), (4, 4)]
        for plan in (steps, diag, mixed):
            for d in (sp.a, sp.b, sp.g):
                for v in d.values():
                    v.fill_(float("nan"))
            sp.enqueue(plan)
            got = _snapshot(sp)
            for k in ref:
                assert torch.equal(got[k], ref[k]), (plan, k)
    finally:
        sp.close()
