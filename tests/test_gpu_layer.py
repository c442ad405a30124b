"""A whole layer shard with the attention core between the projections (QKV, causal attention,
output projection, MLP; then the backward in reverse), through the C ABI, against the same layer
computed by the fp64 oracle from the same seeded inputs; and the projection calls split into their
two halves (the form the layer uses) against the whole calls, bit for bit."""
import pytest
import torch

from comm_overlap_amd import synth
from oracle import attention as A
from oracle import layer as L
import gpu_cases as G

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from comm_overlap_amd import tpslice as T

# two 256-token sequences, 4 query heads over 1 key/value head of 128 dims per rank, SwiGLU MLP
LAYER = synth.custom("layer_core", 950, tokens=512, hidden=512, ffn=2048, tp=2, act="swiglu", bias=False,
                     row_slices=2, col_slices=2, heads=8, kv_heads=2, head_dim=128, backward=True)
SEQ = 256


def _e(*shape, dt=torch.bfloat16):
    return torch.full(shape, float("nan"), dtype=dt, device="cuda")


def test_projection_halves_match_whole_calls():
    w = LAYER
    print(f"[case] projection halves {w.key}", flush=True)
    inp = synth.make_inputs(w)
    d = {k: v.to("cuda").contiguous() for k, v in inp.items()}
    with T.plan_for(w) as p:
        i = p.info
        QKV, Z, Zh = _e(i.tokens, i.qkv_width), _e(i.tokens, i.hidden), _e(i.tokens, i.hidden)
        p.attnproj_fwd(d["X"], d["Wqkv"], None, QKV, d["C"], d["Wo"], Z, Zh)
        QKV2, Z2, Zh2 = _e(i.tokens, i.qkv_width), _e(i.tokens, i.hidden), _e(i.tokens, i.hidden)
        p.attnproj_fwd(d["X"], d["Wqkv"], None, QKV2, None, None, None)
        p.attnproj_fwd(None, None, None, None, d["C"], d["Wo"], Z2, Zh2)
        f32 = torch.float32
        full = dict(dX=_e(i.tokens, i.hidden), dXh=_e(i.tokens, i.hidden), dC=_e(i.tokens, i.ctx_width),
                    dWqkv=_e(i.qkv_width, i.hidden, dt=f32), dWo=_e(i.hidden, i.ctx_width, dt=f32))
        half = {k: torch.full_like(v, float("nan")) for k, v in full.items()}
        p.attnproj_bwd(d["X"], d["Wqkv"], d["dQKV"], d["C"], d["Wo"], d["dY_attn"], full["dX"], full["dC"],
                       full["dWqkv"], full["dWo"], dX_handoff=full["dXh"])
        p.attnproj_bwd(None, None, None, d["C"], d["Wo"], d["dY_attn"], None, half["dC"], None, half["dWo"])
        p.attnproj_bwd(d["X"], d["Wqkv"], d["dQKV"], None, None, None, half["dX"], None, half["dWqkv"], None,
                       dX_handoff=half["dXh"])
        torch.cuda.synchronize()
    assert torch.equal(QKV, QKV2) and torch.equal(Z, Z2) and torch.equal(Zh, Zh2)
    for k in full:
        assert torch.equal(full[k], half[k]), k


def run_layer(p, d, seq_len):
    """One layer step on the GPU: QKV -> attention core -> output projection (hand-off) -> MLP
    (hand-off); backward: MLP -> output projection (dC) -> attention core -> QKV projection."""
    i = p.info
    f32 = torch.float32
    o = dict(QKV=_e(i.tokens, i.qkv_width), C=_e(i.tokens, i.ctx_width), lse=_e(i.tokens, i.q_heads, dt=f32),
             Za=_e(i.tokens, i.hidden), Zah=_e(i.tokens, i.hidden), U=_e(i.tokens, i.n1), Z=_e(i.tokens, i.hidden),
             Zh=_e(i.tokens, i.hidden), dX=_e(i.tokens, i.hidden), dXh=_e(i.tokens, i.hidden),
             dW1=_e(i.n1, i.hidden, dt=f32), dW2=_e(i.hidden, i.ffn_shard, dt=f32), dC=_e(i.tokens, i.ctx_width),
             dWo=_e(i.hidden, i.ctx_width, dt=f32), dQKV=_e(i.tokens, i.qkv_width), dXa=_e(i.tokens, i.hidden),
             dXah=_e(i.tokens, i.hidden), dWqkv=_e(i.qkv_width, i.hidden, dt=f32))
    p.attnproj_fwd(d["X"], d["Wqkv"], None, o["QKV"], None, None, None)
    p.attn_core_fwd(o["QKV"], o["C"], seq_len, lse=o["lse"])
    p.attnproj_fwd(None, None, None, None, o["C"], d["Wo"], o["Za"], o["Zah"])
    p.mlp_fwd(o["Zah"], d["W1"], None, d["W2"], o["Z"], o["U"], o["Zh"])
    p.mlp_bwd(o["Zah"], d["W1"], d["W2"], o["U"], d["dY"], o["dX"], o["dW1"], o["dW2"], dX_handoff=o["dXh"])
    p.attnproj_bwd(None, None, None, o["C"], d["Wo"], d["dY_attn"], None, o["dC"], None, o["dWo"])
    p.attn_core_bwd(o["QKV"], o["C"], o["lse"], o["dC"], o["dQKV"], seq_len)
    p.attnproj_bwd(d["X"], d["Wqkv"], o["dQKV"], None, None, None, o["dXa"], None, o["dWqkv"], None,
                   dX_handoff=o["dXah"])
    return o


def oracle_layer(inp, w, seq_len):
    """The same layer in fp64 from the same seeded inputs (no GPU value enters)."""
    f = L.as_f64
    qh, kvh = w.q_heads_shard, w.kv_heads_shard
    X, Wqkv, Wo, W1, W2 = f(inp["X"]), f(inp["Wqkv"]), f(inp["Wo"]), f(inp["W1"]), f(inp["W2"])
    QKV = X @ Wqkv.T
    C = A.attn_core_fwd(QKV, qh, kvh, 128, seq_len)
    Za = C @ Wo.T
    m = L.mlp_fwd(Za, W1, None, W2, w.act)
    mb = L.mlp_bwd(Za, W1, W2, m["U"], f(inp["dY"]), w.act)
    dYa = f(inp["dY_attn"])
    dC = dYa @ Wo
    dWo = dYa.T @ C
    dQKV = A.attn_core_bwd(QKV, dC, qh, kvh, 128, seq_len)
    return dict(QKV=QKV, C=C, Za=Za, Z=m["Z"], dX=mb["dX"], dW1=mb["dW1"], dW2=mb["dW2"], dC=dC, dWo=dWo,
                dQKV=dQKV, dXa=dQKV @ Wqkv, dWqkv=dQKV.T @ X)


@pytest.mark.parametrize("pipeline", [False, True])
def test_layer_with_attention_core_against_oracle(pipeline):
    """Every output of the layer step against the fp64 layer (each GPU stage rounds its output to
    bf16, the oracle keeps fp64 throughout), the hand-off buffers equal to their sources, and the
    same bits from the joined and the pipelined plan."""
    w = LAYER
    print(f"[case] layer with attention core {w.key} pipeline={pipeline}", flush=True)
    inp = synth.make_inputs(w)
    d = {k: v.to("cuda").contiguous() for k, v in inp.items()}
    with T.plan_for(w, pipeline=pipeline, handoff_rows=pipeline) as p:
        o = run_layer(p, d, SEQ)
        p.handoff_wait()
        torch.cuda.synchronize()
    ref = oracle_layer(inp, w, SEQ)
    for k in ("QKV", "C", "Za", "Z", "dX", "dW1", "dW2", "dC", "dWo", "dQKV", "dXa", "dWqkv"):
        G.assert_parity(o[k], ref[k], k)
    for k in ("Zah", "Zh", "dXh", "dXah"):
        assert torch.equal(o[k], o[k[:-1]]), k
    if pipeline:
        with T.plan_for(w) as j:
            oj = run_layer(j, d, SEQ)
            torch.cuda.synchronize()
        for k in o:
            assert torch.equal(o[k], oj[k]), k
