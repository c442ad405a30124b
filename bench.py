#!/usr/bin/env python3
"""Benchmark of the sliced tensor-parallel layer shard on one MI355X.

A step is one pass of the whole path over one batch. For a forward MLP workload: one
tpslice_mlp_fwd call (column-parallel up-projection with the fused activation, row-parallel
down-projection in pieces, each finished piece handed off by a DMA-engine copy on a side stream).
For a layer workload: the attention projections and the MLP, forward and backward. Steps are
chained the way consecutive layers are (each call reads the previous call's hand-off buffer) and
the plan pipelines the hand-off: row slice i of a call waits only for row slice i of the previous
call's hand-off, so a call's last copies overlap the next call's first products. Inputs are
synthetic, seeded, and resident in HBM before timing starts.

Order of a run: W warm-up steps; R rounds of five legs taken in alternation (the pipelined chain,
the same chain without hand-off copies, the hand-off copies alone, isolated calls with and without
copies), which give the wall form of the hidden copy time from the legs' medians and also bring the
clocks to steady state; then the K timed steps of the headline; then the same K steps traced (every
product's launch timed by HIP events that the dispatches record themselves, on the streams they run
on), and traced again with the copies, for the trace form of the hidden copy time (the share of the
copies' time during which a product ran) in steady state and for isolated calls.

Prints ONE JSON line: TFLOP/s (algorithmic 2*M*N*K flops of every product / wall time of the K
timed steps), the fraction of the dense bf16 MFMA peak, the hidden copy time (trace form as the
headline, wall form beside it), the roofline of the dominant product (the largest share of the
step's product time), and the fp64 CPU oracle timed on the host's cores over a bounded row sample
(a baseline, not a target).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload KEY]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "TFLOP/s and % of bf16 MFMA peak per TP-shard layer; % copy time hidden"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
# The rate register-only MFMA chains reach on this GPU, with no memory traffic (2.44 PFLOP/s at
# 2.39 GHz; comm_overlap_amd/probes/mfma_rate.hip, summary in profiles/mfma_rate.txt): the ceiling
# a kernel of this library can approach, reported beside the published peak.
MFMA_CEILING_TFLOPS = 2440.0
DEFAULT_WORKLOAD = "llama3_70b_layer"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rounds", type=int, default=5,
                    help="rounds of the alternating hand-off legs (wall form of the hidden copy time)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--streams", type=int, default=0, help="worker streams (0 = plan default)")
    ap.add_argument("--copy-streams", type=int, default=0, help="copy streams (0 = plan default)")
    ap.add_argument("--row-slices", type=int, default=0, help="row slices (0 = the workload's)")
    ap.add_argument("--col-slices", type=int, default=0, help="column slices (0 = the workload's)")
    ap.add_argument("--tile", default="auto",
                    choices=["auto", "256x256", "128x128", "256x320", "128x320", "128x256", "128x128w8", "256x256w4",
                             "256x160w4", "256x320w4", "256x224w4", "large", "small"],
                    help="block tile of every product (auto = chosen per product, the default)")
    ap.add_argument("--dh-group", type=int, default=0,
                    help="row slices per dH product of the MLP backward (0 = plan default)")
    ap.add_argument("--up-group", type=int, default=0,
                    help="row slices per up-projection of the MLP forward (0 = plan default)")
    ap.add_argument("--copy-blit", action="store_true", help="hand-off by copy kernel instead of DMA")
    ap.add_argument("--caller-worker", action="store_true",
                    help="worker stream 0 is the caller's stream (plans with one worker stream always do this)")
    ap.add_argument("--handoff-pieces", action="store_true",
                    help="column slices: a 2D copy per (row, column) piece (a copy kernel on the compute units) "
                         "instead of the default one contiguous DMA copy per row slice")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU-oracle time")
    ap.add_argument("--no-strands", action="store_true",
                    help="skip the two-strand leg (layer workloads: forward of one micro-batch beside the backward "
                         "of another, paired by the library's schedule from a measured pairwise profile)")
    ap.add_argument("--strands-exhaustive", action="store_true",
                    help="also measure every pairing of the two strands' segments (the schedule's check)")
    ap.add_argument("--attn-seq", type=int, default=2048,
                    help="sequence length for the attention-core leg of layer workloads")
    ap.add_argument("--no-attn-core", action="store_true", help="skip the attention-core leg")
    ap.add_argument("--no-blas-context", action="store_true",
                    help="skip timing each product's shape with torch.matmul (vendor BLAS) for context")
    ap.add_argument("--calib-copy", action="store_true",
                    help="finish with plain 256 MiB device copies (counter calibration for profiles)")
    return ap.parse_args()


ROOT = os.path.dirname(os.path.abspath(__file__))
CALIB_BYTES = 256 << 20


def recorded_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` (template parameters and grid) from the committed counter
    summary of this workload, if that summary covers this kernel and was taken on the current GEMM
    source (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"gemm_kernel_{workload}_traffic.txt")
    src = os.path.join(ROOT, "comm_overlap_amd", "csrc", "gemm.hip")
    if not os.path.exists(path):
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    fields = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("gemm.hip sha256") != sha or fields.get("kernel") != kernel:
        return None
    if "traffic_bytes_per_launch" not in fields:
        return None
    return float(fields["traffic_bytes_per_launch"])


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class Chain:
    """Device buffers and calls of chained steps. Step n writes hand-off buffer set n % 2 and reads
    the other set as its input, as consecutive layers would. `dev`: the workload's inputs in HBM
    (shared by every chain); `share`: another chain whose activation buffers and gradients this one
    reuses (legs that never run at the same time)."""

    def __init__(self, w, plan, dev, handoff=True, share=None):
        import torch
        self.w, self.plan, self.handoff, self.t = w, plan, handoff, dev
        i = plan.info
        bf, f32 = torch.bfloat16, torch.float32
        e = lambda *s, dt=bf: torch.empty(*s, dtype=dt, device="cuda")
        if share is not None:
            self.sets, self.g = share.sets, share.g
        else:
            self.sets = []
            for _ in range(2):
                o = {"Z": e(i.tokens, i.hidden), "Zh": e(i.tokens, i.hidden), "U": e(i.tokens, i.n1)}
                if w.has_attn:
                    o.update(QKV=e(i.tokens, i.qkv_width), Za=e(i.tokens, i.hidden), Zah=e(i.tokens, i.hidden))
                if w.backward:
                    o.update(dX=e(i.tokens, i.hidden), dXh=e(i.tokens, i.hidden))
                    if w.has_attn:
                        o.update(dXa=e(i.tokens, i.hidden), dXah=e(i.tokens, i.hidden),
                                 dC=e(i.tokens, i.ctx_width))
                self.sets.append(o)
            # the chain's first input is the seeded X; later steps read the previous step's output
            for o in self.sets:
                o["Zh"].copy_(self.t["X" if w.has_attn else "X_mlp"])
                o["Z"].copy_(o["Zh"])
            self.g = {"dW1": e(i.n1, i.hidden, dt=f32), "dW2": e(i.hidden, i.ffn_shard, dt=f32)}
            if w.bias:
                self.g["db1"] = e(i.n1, dt=f32)
            if w.has_attn:
                self.g.update(dWqkv=e(i.qkv_width, i.hidden, dt=f32), dWo=e(i.hidden, i.ctx_width, dt=f32))
        for op in range(4):
            plan.workspace(op)
        self.n = 0

    def handoff_tensors(self):
        """(source, destination) pairs a step hands off."""
        o = self.sets[0]
        pairs = [(o["Z"], o["Zh"])]
        if self.w.has_attn:
            pairs.append((o["Za"], o["Zah"]))
        if self.w.backward:
            pairs.append((o["dX"], o["dXh"]))
            if self.w.has_attn:
                pairs.append((o["dXa"], o["dXah"]))
        return pairs

    def __call__(self):
        w, t, p, g = self.w, self.t, self.plan, self.g
        o, prev = self.sets[self.n % 2], self.sets[(self.n + 1) % 2]
        h = self.handoff
        out = lambda k: o[k] if h else None
        x_prev = prev["Zh"] if h else prev["Z"]
        if w.has_attn:
            p.attnproj_fwd(x_prev, t["Wqkv"], None, o["QKV"], t["C"], t["Wo"], o["Za"], out("Zah"))
            x_mlp = o["Zah"] if h else o["Za"]
        else:
            x_mlp = x_prev
        p.mlp_fwd(x_mlp, t["W1"], t.get("b1"), t["W2"], o["Z"], o["U"], out("Zh"))
        if w.backward:
            p.mlp_bwd(x_mlp, t["W1"], t["W2"], t["U_saved"], t["dY"], o["dX"], g["dW1"], g["dW2"],
                      db1=g.get("db1"), dX_handoff=out("dXh"))
            if w.has_attn:
                dy_attn = o["dXh"] if h else o["dX"]
                p.attnproj_bwd(x_prev, t["Wqkv"], t["dQKV"], t["C"], t["Wo"], dy_attn, o["dXa"], o["dC"],
                               g["dWqkv"], g["dWo"], dX_handoff=out("dXah"))
        self.n += 1


def timed(fn, steps, warmup, plans=()):
    """Wall time per step of `steps` back-to-back calls, bracketed by full synchronization (and by
    waits for the pipelined hand-off copies of `plans`)."""
    import torch
    for _ in range(warmup):
        fn()
    for p in plans:
        p.handoff_wait()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    for p in plans:
        p.handoff_wait()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / max(1, steps)


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def kernel_stats(recs, key):
    """GEMM launches grouped by `key` ("step": the product; "kernel": the kernel's identity, i.e.
    its template parameters and grid, as a kernel profiler groups dispatches)."""
    by = {}
    for r in recs:
        if r["kind"] != "gemm":
            continue
        d = by.setdefault(r[key], {"n": 0, "ms": 0.0, "flops": 0.0, "steps": set(), "grid_x": r["grid_x"]})
        d["n"] += 1
        d["ms"] += r["end_ms"] - r["start_ms"]
        d["flops"] += r["flops"]
        d["steps"].add(r["step"])
    return by


def union(iv):
    out = []
    for s, e in sorted(iv):
        if out and s <= out[-1][1]:
            out[-1][1] = max(out[-1][1], e)
        else:
            out.append([s, e])
    return out


def hidden_from_trace(recs):
    """The trace form of the hidden hand-off: the share of the copies' time during which at least
    one product ran, from the plan's own events (copy intervals from the copy stream reaching the
    copy to the fence after it; product intervals from the dispatches' own timestamps)."""
    busy = union([(r["start_ms"], r["end_ms"]) for r in recs if r["kind"] != "copy"])
    tot = hid = 0.0
    for r in recs:
        if r["kind"] != "copy":
            continue
        s, e = r["start_ms"], r["end_ms"]
        tot += e - s
        for a, b in busy:
            if b <= s:
                continue
            if a >= e:
                break
            hid += min(e, b) - max(s, a)
    return (hid / tot if tot > 0 else None), tot


def core_flops(w, seq_len):
    """Algorithmic flops of the causal attention core over the layer's tokens: per query head and
    sequence, the causal pairs (t >= s: seq_len (seq_len + 1) / 2) times 2 head_dim for each product;
    two products forward (S, PV), four backward (dV, dP, dK, dQ; recomputing S is not counted)."""
    pairs = seq_len * (seq_len + 1) / 2.0
    per = pairs * 2.0 * 128 * w.q_heads_shard * (w.tokens // seq_len)
    return 2.0 * per, 4.0 * per


def product_shapes(w, info):
    """(M, N, K, operand orientation) of each product of a step as one plain matmul: "nt" A @ B^T,
    "nn" A @ B, "tn" A^T @ B (the weight gradients, over all tokens)."""
    M, h, Fp, N1 = info.tokens, info.hidden, info.ffn_shard, info.n1
    Ms = info.rows_per_slice
    out = {"mlp_up": (Ms * info.up_group_slices, N1, h, "nt"), "mlp_down": (Ms, h, Fp, "nt")}
    if w.backward:
        out.update(mlp_dh=(Ms * info.dh_group_slices, Fp, h, "nn"), mlp_dx=(Ms, h, N1, "nn"),
                   mlp_dw1=(N1, h, M, "tn"), mlp_dw2=(h, Fp, M, "tn"))
    if w.has_attn:
        q, c = info.qkv_width, info.ctx_width
        out.update(qkv=(M, q, h, "nt"), out=(Ms, h, c, "nt"))
        if w.backward:
            out.update(attn_dx=(Ms, h, q, "nn"), attn_dc=(M, c, h, "nn"), attn_dwo=(h, c, M, "tn"),
                       attn_dwqkv=(q, h, M, "tn"))
    return out


def blas_context(w, info, kernels):
    """Context, not a target: each product's shape as one torch.matmul in bf16 (the vendor BLAS that
    torch's preferred BLAS library names; bf16 output, where this library's weight gradients write
    fp32), median of 10 timed calls, beside this library's per-launch rate of the same product in
    the traced steps."""
    import torch
    res = {"blas_library": str(torch.backends.cuda.preferred_blas_library()).split(".")[-1]}
    for name, (M, N, K, form) in product_shapes(w, info).items():
        if name not in kernels:
            continue
        a = torch.randn(K, M, device="cuda").to(torch.bfloat16) if form == "tn" else \
            torch.randn(M, K, device="cuda").to(torch.bfloat16)
        b = torch.randn(N, K, device="cuda").to(torch.bfloat16) if form == "nt" else \
            torch.randn(K, N, device="cuda").to(torch.bfloat16)
        fn = {"nt": lambda: torch.matmul(a, b.t()), "nn": lambda: torch.matmul(a, b),
              "tn": lambda: torch.matmul(a.t(), b)}[form]
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[len(ts) // 2]
        res[name] = {"shape": [M, N, K], "torch_matmul_tflops": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1),
                     "tpslice_tflops": kernels[name]["tflops"]}
        del a, b
    torch.cuda.synchronize()
    return res


def attn_core(w, inp, seq_len, steps):
    """The causal attention core between the projections (tpslice_attn_core_fwd and _bwd) over the
    layer's tokens as sequences of seq_len rows, each timed alone on the caller's stream."""
    import torch
    from comm_overlap_amd import synth
    from comm_overlap_amd import tpslice as T
    if w.tokens % seq_len:
        return None
    plan = T.plan_for(w)
    i = plan.info
    qkv = synth.randn_bf16((w.tokens, w.qkv_width), 1.0, 7).cuda()
    dc = synth.randn_bf16((w.tokens, i.ctx_width), 1.0, 8).cuda()
    c = torch.empty(w.tokens, i.ctx_width, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(w.tokens, i.q_heads, dtype=torch.float32, device="cuda")
    dqkv = torch.empty_like(qkv)
    plan.workspace(T.OP_ATTN_CORE_BWD)
    fwd = lambda: plan.attn_core_fwd(qkv, c, seq_len, lse=lse)
    bwd = lambda: plan.attn_core_bwd(qkv, c, lse, dc, dqkv, seq_len)
    out = {"seq_len": seq_len, "q_heads": w.q_heads_shard, "kv_heads": w.kv_heads_shard, "head_dim": 128}
    fl = dict(zip(("fwd", "bwd"), core_flops(w, seq_len)))
    for name, fn in (("fwd", fwd), ("bwd", bwd)):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = max(10, steps)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        tf = fl[name] / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    plan.close()
    return out


class LayerWithCore:
    """The whole layer step with the attention core between the projections: QKV, the core, the
    output projection (hand-off) and the MLP (hand-off); backward: the MLP, the output projection's
    dC, the core's backward and the QKV projection's dX (hand-off) and weight gradients. Steps are
    chained as in Chain (each reads the previous step's hand-off)."""

    def __init__(self, w, plan, dev, seq_len):
        import torch
        self.w, self.p, self.t, self.seq = w, plan, dev, seq_len
        i = plan.info
        bf, f32 = torch.bfloat16, torch.float32
        e = lambda *s, dt=bf: torch.empty(*s, dtype=dt, device="cuda")
        self.sets = []
        for _ in range(2):
            self.sets.append(dict(QKV=e(i.tokens, i.qkv_width), C=e(i.tokens, i.ctx_width),
                                  lse=e(i.tokens, i.q_heads, dt=f32), Za=e(i.tokens, i.hidden),
                                  Zah=e(i.tokens, i.hidden), U=e(i.tokens, i.n1), Z=e(i.tokens, i.hidden),
                                  Zh=e(i.tokens, i.hidden), dX=e(i.tokens, i.hidden), dXh=e(i.tokens, i.hidden),
                                  dC=e(i.tokens, i.ctx_width), dQKV=e(i.tokens, i.qkv_width),
                                  dXa=e(i.tokens, i.hidden), dXah=e(i.tokens, i.hidden)))
        for o in self.sets:
            o["Zh"].copy_(dev["X"])
        self.g = dict(dW1=e(i.n1, i.hidden, dt=f32), dW2=e(i.hidden, i.ffn_shard, dt=f32),
                      dWo=e(i.hidden, i.ctx_width, dt=f32), dWqkv=e(i.qkv_width, i.hidden, dt=f32))
        for op in range(5):
            plan.workspace(op)
        self.n = 0

    def __call__(self):
        p, t, g, s = self.p, self.t, self.g, self.seq
        o, prev = self.sets[self.n % 2], self.sets[(self.n + 1) % 2]
        x = prev["Zh"]
        p.attnproj_fwd(x, t["Wqkv"], None, o["QKV"], None, None, None)
        p.attn_core_fwd(o["QKV"], o["C"], s, lse=o["lse"])
        p.attnproj_fwd(None, None, None, None, o["C"], t["Wo"], o["Za"], o["Zah"])
        p.mlp_fwd(o["Zah"], t["W1"], t.get("b1"), t["W2"], o["Z"], o["U"], o["Zh"])
        p.mlp_bwd(o["Zah"], t["W1"], t["W2"], o["U"], t["dY"], o["dX"], g["dW1"], g["dW2"], dX_handoff=o["dXh"])
        p.attnproj_bwd(None, None, None, o["C"], t["Wo"], o["dXh"], None, o["dC"], None, g["dWo"])
        p.attn_core_bwd(o["QKV"], o["C"], o["lse"], o["dC"], o["dQKV"], s)
        p.attnproj_bwd(x, t["Wqkv"], o["dQKV"], None, None, None, o["dXa"], None, g["dWqkv"], None,
                       dX_handoff=o["dXah"])
        self.n += 1


def cpu_baseline(w, inp, target_s):
    """The fp64 oracle, as it stands, on the host's cores over a bounded row sample of the workload."""
    from oracle import layer as L
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    f64 = L.as_f64
    M = w.tokens
    fl_full = sum(w.gemm_flops().values())
    # rows are independent: a row sample costs rows/M of the full workload; size it from a probe
    probe_rows = max(64, min(M, 512))
    X = f64(inp["X_mlp"][:probe_rows])
    t0 = time.perf_counter()
    L.mlp_fwd(X, f64(inp["W1"]), f64(inp["b1"]) if "b1" in inp else None, f64(inp["W2"]), w.act)
    rate = 2.0 * probe_rows * w.hidden * (w.n1 + w.ffn_shard) / max(1e-6, time.perf_counter() - t0)
    rows = int(min(M, max(64, target_s * rate / (fl_full / M))) // 64 * 64) or 64
    sel = slice(0, rows)
    A = {k: f64(v[sel]) if v.dim() == 2 and v.shape[0] == M else f64(v) for k, v in inp.items()}

    def run():
        L.mlp_fwd(A["X_mlp"], A["W1"], A.get("b1"), A["W2"], w.act)
        if w.has_attn:
            L.attnproj_fwd(A["X"], A["Wqkv"], None, A["C"], A["Wo"])
        if w.backward:
            L.mlp_bwd(A["X_mlp"], A["W1"], A["W2"], A["U_saved"], A["dY"], w.act, with_bias=w.bias)
            if w.has_attn:
                L.attnproj_bwd(A["X"], A["Wqkv"], A["dQKV"], A["C"], A["Wo"], A["dY_attn"])

    t0 = time.perf_counter()
    reps = 0
    while True:
        run()
        reps += 1
        t = time.perf_counter() - t0
        if t >= 0.8 * target_s or reps >= 20:
            break
    flops = fl_full * rows / M * reps
    return {"value": round(flops / t / 1e12, 4), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows} of {M} token rows of the same workload (all its products), fp64 NumPy "
                      f"(OpenBLAS), {reps} run(s) in {t:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported. The path is one GPU's "
              f"tensor-parallel share; across GPUs each rank would run it on its own weight shards and "
              f"sum the hand-off pieces with a collective on the copy stream.", file=sys.stderr)
        return 2
    import torch
    from comm_overlap_amd import synth
    from comm_overlap_amd import tpslice as T

    w = synth.WORKLOADS[args.workload]
    log(f"workload {w.key}: generating inputs")
    inp = synth.make_inputs(w)
    dev = {k: v.to("cuda").contiguous() for k, v in inp.items()}
    flops = sum(w.gemm_flops().values())
    kw = dict(n_streams=args.streams, n_copy_streams=args.copy_streams, copy_blit=args.copy_blit, tile=args.tile,
              handoff_rows=not args.handoff_pieces, caller_worker=args.caller_worker, dh_group=args.dh_group,
              up_group=args.up_group)
    if args.row_slices:
        kw["n_row_slices"] = args.row_slices
    if args.col_slices:
        kw["n_col_slices"] = args.col_slices
    plan = T.plan_for(w, pipeline=True, **kw)  # the headline: chained steps, pipelined hand-off
    jplan = T.plan_for(w, **kw)                # every call joined: isolated calls
    # the copies alone: every piece's copy back to back behind a one-worker plan's events, so that the
    # time is the copies' own (a plan with more worker streams adds event hops between them)
    cplan = T.plan_for(w, **dict(kw, n_streams=1))
    chain = Chain(w, plan, dev)
    nocopy = Chain(w, plan, dev, handoff=False, share=chain)
    jchain = Chain(w, jplan, dev, share=chain)
    jnocopy = Chain(w, jplan, dev, handoff=False, share=chain)
    pairs = chain.handoff_tensors()

    def copies():
        for s, d in pairs:
            cplan.handoff_copy(s, d)

    torch.cuda.synchronize()
    K = args.steps
    log(f"warmup {args.warmup}")
    timed(chain, 0, args.warmup, [plan])

    # 1) the wall form of the hidden hand-off, from legs taken in alternation over several rounds
    # (medians): the pipelined chain, the same chain without hand-off copies, the copies alone, and
    # the same pair for isolated (joined) calls. These legs also bring the clocks to steady state
    # before the headline.
    rounds = max(1, args.rounds)
    log(f"hand-off legs: {rounds} rounds x 5 legs x {K} steps")
    legs = {k: [] for k in ("chain", "nocopy", "copies", "iso", "iso_nocopy")}
    for _ in range(rounds):
        legs["chain"].append(timed(chain, K, 1, [plan]))
        legs["nocopy"].append(timed(nocopy, K, 1, [plan]))
        legs["copies"].append(timed(copies, K, 1, [cplan]))
        legs["iso"].append(timed(jchain, K, 1))
        legs["iso_nocopy"].append(timed(jnocopy, K, 1))
    med = {k: median(v) for k, v in legs.items()}
    hw = lambda a, b: max(0.0, min(1.0, 1.0 - (a - b) / med["copies"])) if med["copies"] > 0 else None
    hidden_wall = hw(med["chain"], med["nocopy"])
    hidden_wall_single = hw(med["iso"], med["iso_nocopy"])

    # 2) headline: K chained steps with the pipelined hand-off, untraced
    log(f"timed region: {K} steps")
    ms = timed(chain, K, 0, [plan])

    # 3) the same K steps with every product's launch timed by HIP events that the dispatches record
    # themselves, on the streams they run on: the roofline's per-launch durations
    log(f"traced pass (products): {K} steps")
    plan.trace(True, products=True, copies=False)
    ms_traced = timed(chain, K, 0, [plan])
    recs = plan.trace_read()
    by = kernel_stats(recs, "step")
    by_kernel = kernel_stats(recs, "kernel")
    # 4) products and copies traced: the trace form of the hidden hand-off, in steady state (the
    # pipelined chain) and for isolated calls (each call joined)
    log(f"traced pass (products and copies): {K} steps, chained and isolated")
    plan.trace(True, products=True, copies=True)
    timed(chain, K, 0, [plan])
    hidden_trace, copy_ms = hidden_from_trace(plan.trace_read())
    plan.trace(False)
    jplan.trace(True, products=True, copies=True)
    timed(jchain, K, 0)
    hidden_trace_single, _ = hidden_from_trace(jplan.trace_read())
    jplan.trace(False)
    info = plan.info

    # 5) two strands (layer workloads): the forward of one micro-batch beside the backward of another,
    # in segments of half a micro-batch; the pairwise profile P measured here, the pairing chosen by
    # the library's schedule, then measured; the same segments in sequence for comparison
    two = None
    if w.has_attn and w.backward and not args.no_strands:
        from comm_overlap_amd import strands as ST
        log("two strands: pairwise profile, schedule, measured pairing")
        sp = ST.StrandPair(w, dev, dict(tile=args.tile, copy_blit=args.copy_blit))
        P = sp.profile(reps=3)
        plan_steps, predicted = ST.schedule(P)
        measured = sp.time(plan_steps, reps=5)
        seq_ms = sp.time(sp.sequential(), reps=5)
        two = {"segments": {"forward": ["attnproj_fwd half 1", "attnproj_fwd half 2", "mlp_fwd half 1",
                                        "mlp_fwd half 2"],
                            "backward": ["mlp_bwd half 1", "mlp_bwd half 2", "attnproj_bwd half 1",
                                         "attnproj_bwd half 2"]},
               "P_ms": [[round(x, 4) for x in row] for row in P], "plan": plan_steps,
               "predicted_ms": round(predicted, 4), "measured_ms": round(measured, 4),
               "sequential_ms": round(seq_ms, 4), "speedup_vs_sequential": round(seq_ms / measured, 3),
               "tflops": round(flops / (measured * 1e-3) / 1e12, 2)}
        if args.strands_exhaustive:
            log("two strands: every pairing")
            allp = ST.pairings(len(sp.fwd), len(sp.bwd))
            meas = [(sp.time(s, reps=3), s) for s in allp]
            meas.sort(key=lambda x: x[0])
            pred = {tuple(s): sum(P[i][j] for i, j in s) for s in allp}
            rank = next(k for k, (_, s) in enumerate(meas) if s == plan_steps)
            errs = sorted(abs(m - pred[tuple(s)]) / m for m, s in meas)
            two["exhaustive"] = {"pairings": len(allp), "best_measured_ms": round(meas[0][0], 4),
                                 "best_plan": meas[0][1], "schedule_rank": rank,
                                 "schedule_vs_best": round(measured / meas[0][0], 4),
                                 "median_prediction_error": round(errs[len(errs) // 2], 4),
                                 "max_prediction_error": round(errs[-1], 4)}
        sp.close()
        del sp

    # 6) the whole layer with the attention core between the projections (layer workloads)
    layer_core = None
    if w.has_attn and w.backward and not args.no_attn_core and w.tokens % args.attn_seq == 0:
        log("layer step with the attention core")
        lc = LayerWithCore(w, plan, dev, args.attn_seq)
        ms_lc = timed(lc, K, 2, [plan])
        cf, cb = core_flops(w, args.attn_seq)
        fl_lc = flops + cf + cb
        layer_core = {"seq_len": args.attn_seq, "ms_per_step": round(ms_lc, 4),
                      "tflops": round(fl_lc / (ms_lc * 1e-3) / 1e12, 2),
                      "pct_of_peak": round(100.0 * fl_lc / (ms_lc * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                      "gflop_per_step": round(fl_lc / 1e9, 1), "core_gflop_per_step": round((cf + cb) / 1e9, 1)}
        del lc

    tflops = flops / (ms * 1e-3) / 1e12
    # the dominant kernel: the GEMM kernel (template parameters and grid) with the largest share of
    # the step's product time; its launches may serve more than one product of that grid
    dom_name, dom = max(by_kernel.items(), key=lambda kv: kv[1]["ms"])
    dom_ms = dom["ms"] / dom["n"]
    achieved = dom["flops"] / dom["n"] / (dom_ms * 1e-3) / 1e12
    pct = lambda x: None if x is None else round(100.0 * x, 1)
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.key, "tokens": w.tokens, "hidden": w.hidden, "ffn_shard": w.ffn_shard,
                   "tp_share": f"1/{w.tp}", "act": w.act, "row_slices": info.n_row_slices,
                   "col_slices": info.n_col_slices, "backward": w.backward,
                   "heads_shard": [w.q_heads_shard, w.kv_heads_shard] if w.has_attn else None,
                   "worker_streams": info.n_streams, "copy_streams": info.n_copy_streams,
                   "up_group_slices": info.up_group_slices,
                   "dh_group_slices": info.dh_group_slices if w.backward else None,
                   "tile": args.tile,
                   "handoff": "blit" if args.copy_blit else (
                       "dma, whole row slices" if not args.handoff_pieces and info.n_col_slices > 1
                       else "dma"), "chain": "pipelined"},
        "pct_of_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "pct_of_mfma_ceiling": round(100.0 * tflops / MFMA_CEILING_TFLOPS, 2),
        "hidden_copy_pct": pct(hidden_trace),
        "hidden_copy_pct_single_call": pct(hidden_trace_single),
        "hidden_copy_wall_pct": pct(hidden_wall),
        "hidden_copy_wall_pct_single_call": pct(hidden_wall_single),
        "handoff_copy_ms_per_step_traced": round(copy_ms / max(1, K), 4),
        "legs_ms_median": {k: round(v, 4) for k, v in med.items()},
        "legs_rounds": rounds,
        "ms_per_step_traced": round(ms_traced, 4),
        "roofline": {"bound": "mfma", "kernel": dom_name, "products": sorted(dom["steps"]),
                     "grid_x": dom["grid_x"], "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(w.key, dom_name), "launches_per_step": dom["n"] / K,
                     "avg_launch_ms": round(dom_ms, 4), "flops_per_launch": dom["flops"] / dom["n"]},
        "kernels": {k: {"launches": v["n"], "avg_ms": round(v["ms"] / v["n"], 4),
                        "tflops": round(v["flops"] / (v["ms"] * 1e-3) / 1e12, 1)} for k, v in by.items()},
    }
    if two is not None:
        out["two_strands"] = two
    if layer_core is not None:
        out["layer_with_attention_core"] = layer_core
    if w.has_attn and not args.no_attn_core:
        log("attention core")
        out["attn_core"] = attn_core(w, inp, args.attn_seq, K)
    if not args.no_blas_context:
        log("vendor BLAS context")
        out["blas_context"] = blas_context(w, info, out["kernels"])
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle)")
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    plan.handoff_wait()
    torch.cuda.synchronize()
    if args.calib_copy:
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)  # elementwise kernel: reads and writes CALIB_BYTES
        torch.cuda.synchronize()
    plan.close()
    jplan.close()
    cplan.close()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
