"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI on seeded inputs and
compute the oracle's answer for the same inputs (whole tensors, or sampled rows/columns)."""
from __future__ import annotations

import numpy as np
import torch

from comm_overlap_amd import synth
from oracle import layer as L
from oracle.compare import compare

f64 = L.as_f64


def dev(t):
    return None if t is None else t.to("cuda", non_blocking=False).contiguous()


def host(t):
    return t.detach().to("cpu")


def assert_parity(g, o, name):
    v = compare(f64(g), o, name)
    assert v.ok, str(v)
    return v


def run_mlp_fwd(plan, inp, save_u=True, handoff=True, sync=True):
    X, W1, W2 = dev(inp["X_mlp"]), dev(inp["W1"]), dev(inp["W2"])
    b1 = dev(inp.get("b1"))
    i = plan.info
    Z = torch.full((i.tokens, i.hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
    U = torch.empty((i.tokens, i.n1), dtype=torch.bfloat16, device="cuda") if save_u else None
    Zh = torch.full_like(Z, float("nan")) if handoff else None
    plan.mlp_fwd(X, W1, b1, W2, Z, U, Zh)
    if sync:
        torch.cuda.synchronize()
    return {"Z": Z, "U": U, "Zh": Zh}


def oracle_mlp_fwd(inp, act, rows=None):
    X = inp["X_mlp"] if rows is None else inp["X_mlp"][rows]
    return L.mlp_fwd(f64(X), f64(inp["W1"]), f64(inp["b1"]) if "b1" in inp else None, f64(inp["W2"]), act)


def run_attn_fwd(plan, inp, handoff=True, bias=None, sync=True):
    i = plan.info
    QKV = torch.empty((i.tokens, i.qkv_width), dtype=torch.bfloat16, device="cuda")
    Z = torch.empty((i.tokens, i.hidden), dtype=torch.bfloat16, device="cuda")
    Zh = torch.empty_like(Z) if handoff else None
    plan.attnproj_fwd(dev(inp["X"]), dev(inp["Wqkv"]), dev(bias), QKV, dev(inp["C"]), dev(inp["Wo"]), Z, Zh)
    if sync:
        torch.cuda.synchronize()
    return {"QKV": QKV, "Z": Z, "Zh": Zh}


def run_mlp_bwd(plan, inp, with_bias, handoff=True, accumulate=False, init=None, sync=True):
    i = plan.info
    dX = torch.empty((i.tokens, i.hidden), dtype=torch.bfloat16, device="cuda")
    dXh = torch.empty_like(dX) if handoff else None
    if init is None:
        dW1 = torch.empty((i.n1, i.hidden), dtype=torch.float32, device="cuda")
        dW2 = torch.empty((i.hidden, i.ffn_shard), dtype=torch.float32, device="cuda")
        db1 = torch.empty((i.n1,), dtype=torch.float32, device="cuda") if with_bias else None
    else:
        dW1, dW2, db1 = (None if t is None else t.clone() for t in init)
    plan.mlp_bwd(dev(inp["X_mlp"]), dev(inp["W1"]), dev(inp["W2"]), dev(inp["U_saved"]), dev(inp["dY"]),
                 dX, dW1, dW2, db1=db1, dX_handoff=dXh, accumulate=accumulate)
    if sync:
        torch.cuda.synchronize()
    return {"dX": dX, "dXh": dXh, "dW1": dW1, "dW2": dW2, "db1": db1}


def run_attn_bwd(plan, inp, with_bias, handoff=True, accumulate=False, init=None, sync=True):
    i = plan.info
    dX = torch.empty((i.tokens, i.hidden), dtype=torch.bfloat16, device="cuda")
    dXh = torch.empty_like(dX) if handoff else None
    dC = torch.empty((i.tokens, i.ctx_width), dtype=torch.bfloat16, device="cuda")
    if init is None:
        dWqkv = torch.empty((i.qkv_width, i.hidden), dtype=torch.float32, device="cuda")
        dWo = torch.empty((i.hidden, i.ctx_width), dtype=torch.float32, device="cuda")
        dbqkv = torch.empty((i.qkv_width,), dtype=torch.float32, device="cuda") if with_bias else None
    else:
        dWqkv, dWo, dbqkv = (None if t is None else t.clone() for t in init)
    plan.attnproj_bwd(dev(inp["X"]), dev(inp["Wqkv"]), dev(inp["dQKV"]), dev(inp["C"]), dev(inp["Wo"]),
                      dev(inp["dY_attn"]), dX, dC, dWqkv, dWo, dbqkv=dbqkv, dX_handoff=dXh,
                      accumulate=accumulate)
    if sync:
        torch.cuda.synchronize()
    return {"dX": dX, "dXh": dXh, "dC": dC, "dWqkv": dWqkv, "dWo": dWo, "dbqkv": dbqkv}


def sample_rows(M, r, per_slice=8, seed=0):
    """Rows from every row slice, including each slice's first and last row."""
    rng = np.random.default_rng(seed)
    Ms = M // r
    rows = []
    for i in range(r):
        rows += [i * Ms, (i + 1) * Ms - 1]
        rows += list(rng.integers(i * Ms, (i + 1) * Ms, per_slice - 2))
    return np.array(sorted(set(int(x) for x in rows)))


def sample_cols(n, k=8, seed=1):
    rng = np.random.default_rng(seed)
    return np.array(sorted(set([0, n - 1] + [int(x) for x in rng.integers(0, n, k - 2)])))


def workload_inputs(w: synth.Workload):
    return synth.make_inputs(w)
