"""Two strands of one layer shard on one GPU: the forward of one micro-batch beside the backward of
another, paired segment by segment (the strand interleaving of the micro-batch co-execution review,
"What carries the argument"; its planner adds up offline pairwise times and picks the pairing by the
recurrence that tpslice_strand_schedule implements).

Segments are calls of the C ABI over half of a micro-batch's tokens (the row slices of one half),
in each strand's own order:
  forward  (micro-batch a): attention projections on half 1, on half 2, MLP forward on half 1, half 2
  backward (micro-batch b): MLP backward on half 1, half 2, attention-projection backward on half 1,
                            half 2 (weight gradients: the second half adds to the first)
Each strand has plans and streams of its own (its caller stream, one copy stream), so that the two
strands' products and hand-off copies can run side by side. A step of a pairing runs one segment
alone or one of each strand at once; every step starts when both strands have finished the step
before. This module only orders calls and events: all arithmetic runs in the library's kernels.
"""
from __future__ import annotations

from typing import Callable, List, Optional, Sequence, Tuple

import torch

from . import tpslice as T

Step = Tuple[int, int]


class StrandPair:
    def __init__(self, w, dev, kw=None, halves: int = 2):
        if not (w.has_attn and w.backward):
            raise ValueError("two strands need a layer workload with attention projections and backward")
        if w.tokens % halves or w.row_slices % halves:
            raise ValueError(f"{halves} parts must divide the tokens and the row slices")
        kw = dict(kw or {})
        kw.update(n_row_slices=w.row_slices // halves, n_col_slices=w.col_slices, n_streams=1, n_copy_streams=1,
                  caller_worker=True)
        self.w, self.t, self.halves = w, dev, halves
        M, h = w.tokens, w.hidden
        self.rows = M // halves
        sub = dict(tokens=self.rows, hidden=h, ffn=w.ffn, tp_size=w.tp, n_heads=w.heads, n_kv_heads=w.kv_heads,
                   head_dim=w.head_dim, act=w.act, handoff_rows=True)
        sub.update(kw)
        self.sa, self.sb = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
        self.gate = torch.cuda.Stream()
        self.pf = T.Plan(T.Config(**sub), T.Streams.new(0, 1))
        self.pb = T.Plan(T.Config(**sub), T.Streams.new(0, 1))
        for p in (self.pf, self.pb):
            for op in range(4):
                p.workspace(op)
        i = self.pf.info
        bf, f32 = torch.bfloat16, torch.float32
        e = lambda *s, dt=bf: torch.empty(*s, dtype=dt, device="cuda")
        self.a = dict(QKV=e(M, i.qkv_width), Za=e(M, h), Zah=e(M, h), Z=e(M, h), Zh=e(M, h), U=e(M, i.n1))
        self.b = dict(dX=e(M, h), dXh=e(M, h), dXa=e(M, h), dXah=e(M, h), dC=e(M, i.ctx_width))
        self.g = dict(dW1=e(i.n1, h, dt=f32), dW2=e(h, i.ffn_shard, dt=f32), dWqkv=e(i.qkv_width, h, dt=f32),
                      dWo=e(h, i.ctx_width, dt=f32))
        self.fwd: List[Callable[[], None]] = ([self._attn_fwd(k) for k in range(halves)]
                                              + [self._mlp_fwd(k) for k in range(halves)])
        self.bwd: List[Callable[[], None]] = ([self._mlp_bwd(k) for k in range(halves)]
                                              + [self._attn_bwd(k) for k in range(halves)])

    # ----------------------------------------------------------------------------- segments
    def _r(self, x, k):
        return x[k * self.rows:(k + 1) * self.rows]

    def _attn_fwd(self, k):
        t, a, r = self.t, self.a, self._r
        return lambda: self.pf.attnproj_fwd(r(t["X"], k), t["Wqkv"], None, r(a["QKV"], k), r(t["C"], k), t["Wo"],
                                            r(a["Za"], k), r(a["Zah"], k))

    def _mlp_fwd(self, k):
        t, a, r = self.t, self.a, self._r
        return lambda: self.pf.mlp_fwd(r(a["Zah"], k), t["W1"], t.get("b1"), t["W2"], r(a["Z"], k), r(a["U"], k),
                                       r(a["Zh"], k))

    def _mlp_bwd(self, k):
        t, b, g, r = self.t, self.b, self.g, self._r
        return lambda: self.pb.mlp_bwd(r(t["X_mlp"], k), t["W1"], t["W2"], r(t["U_saved"], k), r(t["dY"], k),
                                       r(b["dX"], k), g["dW1"], g["dW2"], db1=g.get("db1"),
                                       dX_handoff=r(b["dXh"], k), accumulate=k > 0)

    def _attn_bwd(self, k):
        t, b, g, r = self.t, self.b, self.g, self._r
        return lambda: self.pb.attnproj_bwd(r(t["X"], k), t["Wqkv"], r(t["dQKV"], k), r(t["C"], k), t["Wo"],
                                            r(b["dXh"], k), r(b["dXa"], k), r(b["dC"], k), g["dWqkv"], g["dWo"],
                                            dX_handoff=r(b["dXah"], k), accumulate=k > 0)

    # ------------------------------------------------------------------------------ execution
    def enqueue(self, steps: Sequence[Step]):
        """Queue a pairing: each step's forward segment on stream a and backward segment on stream b,
        then a barrier (each stream waits for the other's end of the step)."""
        for i, j in steps:
            if i:
                with torch.cuda.stream(self.sa):
                    self.fwd[i - 1]()
            if j:
                with torch.cuda.stream(self.sb):
                    self.bwd[j - 1]()
            ea, eb = torch.cuda.Event(), torch.cuda.Event()
            ea.record(self.sa)
            eb.record(self.sb)
            self.sa.wait_event(eb)
            self.sb.wait_event(ea)

    def time(self, steps: Sequence[Step], reps: int = 3, gate_cycles: int = 20_000_000) -> float:
        """Median GPU time (ms) of a pairing, from the moment both streams are released to the end of
        its last step. Both streams wait behind a spin kernel on a third stream while the host queues
        the pairing, so that queueing time does not delay one strand against the other."""
        out = []
        for _ in range(reps + 1):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(self.gate):
                torch.cuda._sleep(gate_cycles)
                e0.record(self.gate)
            self.sa.wait_event(e0)
            self.sb.wait_event(e0)
            self.enqueue(steps)
            e1.record(self.sa)  # stream a has waited for stream b's end of the last step
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        out = sorted(out[1:])
        return out[len(out) // 2]

    def profile(self, reps: int = 3) -> List[List[float]]:
        """P[i][j] (ms): forward segment i beside backward segment j, P[i][0] / P[0][j] alone."""
        nf, nb = len(self.fwd), len(self.bwd)
        P = [[0.0] * (nb + 1) for _ in range(nf + 1)]
        for i in range(nf + 1):
            for j in range(nb + 1):
                if i or j:
                    P[i][j] = self.time([(i, j)], reps)
        return P

    def sequential(self) -> List[Step]:
        return [(i + 1, 0) for i in range(len(self.fwd))] + [(0, j + 1) for j in range(len(self.bwd))]

    def close(self):
        torch.cuda.synchronize()
        self.pf.close()
        self.pb.close()


def schedule(P) -> Tuple[List[Step], float]:
    """The library's pairing of least predicted time for the profile P."""
    return T.strand_schedule(P)


def pairings(nf: int, nb: int) -> List[List[Step]]:
    """Every pairing of nf forward and nb backward segments (for the exhaustive measurement)."""
    out: List[List[Step]] = []

    def walk(i, j, path):
        if i == nf and j == nb:
            out.append(list(path))
            return
        for di, dj in ((1, 0), (0, 1), (1, 1)):
            if i + di <= nf and j + dj <= nb:
                path.append((i + 1 if di else 0, j + 1 if dj else 0))
                walk(i + di, j + dj, path)
                path.pop()

    walk(0, 0, [])
    return out
