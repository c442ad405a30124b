"""GPU parity of the causal attention core (through the C ABI) against the fp64 oracle: several
tiles of queries and keys per sequence, several sequences, grouped and ungrouped KV heads, and one
whole sequence of each layer workload's shape."""
import numpy as np
import pytest
import torch

from comm_overlap_amd import synth
from oracle import attention as A
from oracle import layer as L
import gpu_cases as G

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from comm_overlap_amd import tpslice as T


def _case(name, **kw):
    print(f"[case] attn_core {name} {kw}", flush=True)


def _run(w, QKV, seq_len):
    plan = T.plan_for(w)
    i = plan.info
    C = torch.full((i.tokens, i.ctx_width), float("nan"), dtype=torch.bfloat16, device="cuda")
    plan.attn_core_fwd(G.dev(QKV), C, seq_len)
    torch.cuda.synchronize()
    return plan, C


# (tokens, seq_len, heads, kv_heads, tp): q/kv heads per rank = heads/tp, max(1, kv_heads/tp)
# the first and last cases take the paired dealing of query blocks (the last with pairs that straddle
# heads), the others the one-block-per-workgroup order
SMALL = [(512, 256, 8, 2, 2), (384, 128, 5, 5, 1), (256, 256, 8, 8, 8), (640, 128, 16, 2, 2), (2048, 1024, 5, 5, 1)]


@pytest.mark.parametrize("tokens,seq_len,heads,kv_heads,tp", SMALL)
def test_attention_core_small(tokens, seq_len, heads, kv_heads, tp):
    w = synth.custom("attn_core", 930, tokens=tokens, hidden=256, ffn=64, tp=tp, act="gelu", bias=False,
                     row_slices=1, col_slices=1, heads=heads, kv_heads=kv_heads, head_dim=128)
    _case("small", tokens=tokens, seq_len=seq_len, q=w.q_heads_shard, kv=w.kv_heads_shard)
    QKV = synth.randn_bf16((tokens, w.qkv_width), 1.0, 931)
    plan, C = _run(w, QKV, seq_len)
    ref = A.attn_core_fwd(L.as_f64(QKV), w.q_heads_shard, w.kv_heads_shard, 128, seq_len)
    G.assert_parity(C, ref, "C")
    # the same call again gives the same bits; a sequence alone gives its rows of the batch
    _, C2 = _run(w, QKV, seq_len)
    assert torch.equal(C, C2)
    if tokens // seq_len > 1:
        w1 = synth.custom("attn_core1", 930, tokens=seq_len, hidden=256, ffn=64, tp=tp, act="gelu", bias=False,
                          row_slices=1, col_slices=1, heads=heads, kv_heads=kv_heads, head_dim=128)
        _, C1 = _run(w1, QKV[-seq_len:].contiguous(), seq_len)
        assert torch.equal(C1, C[-seq_len:])


def test_attention_core_closed_forms():
    """First token of a sequence: C = its own V, to bf16 rounding. Zero keys: C[t] = mean of V[0..t]."""
    w = synth.custom("attn_cf", 932, tokens=256, hidden=256, ffn=64, tp=2, act="gelu", bias=False,
                     row_slices=1, col_slices=1, heads=8, kv_heads=2, head_dim=128)
    qh, kvh = w.q_heads_shard, w.kv_heads_shard
    QKV = synth.randn_bf16((256, w.qkv_width), 1.0, 933)
    QKV[:, qh * 128:(qh + kvh) * 128] = 0
    _, C = _run(w, QKV, 128)
    Cf = C.float().cpu().numpy().reshape(256, qh, 128)
    V = L.as_f64(QKV)[:, (qh + kvh) * 128:].reshape(256, kvh, 128)
    for b in range(2):
        for h in range(qh):
            g = h // (qh // kvh)
            np.testing.assert_array_equal(Cf[b * 128, h], V[b * 128, g].astype(np.float32))
            mean = np.cumsum(V[b * 128:(b + 1) * 128, g], axis=0) / np.arange(1, 129)[:, None]
            np.testing.assert_allclose(Cf[b * 128:(b + 1) * 128, h], mean, rtol=2e-2, atol=2e-2)


@pytest.mark.parametrize("key", ["llama2_13b_layer", "llama3_70b_layer"])
def test_attention_core_workload_sequence(key):
    """The workload's shard shape (head_dim 128, its query and KV heads per rank) at sequences of 2048
    tokens: every row of the last sequence against the oracle."""
    w = synth.WORKLOADS[key]
    seq = 2048
    _case("workload", key=key, tokens=w.tokens, seq_len=seq)
    QKV = synth.randn_bf16((w.tokens, w.qkv_width), 1.0, 934)
    _, C = _run(w, QKV, seq)
    ref = A.attn_core_fwd(L.as_f64(QKV[-seq:]), w.q_heads_shard, w.kv_heads_shard, 128, seq)
    G.assert_parity(C[-seq:], ref, "C (last sequence)")


# ------------------------------------------------------------------------------------- backward
def _run_bwd(w, QKV, dC, seq_len):
    """Forward with the row log-sum-exp, then the backward; (C, lse, dQKV) on the GPU."""
    plan = T.plan_for(w)
    i = plan.info
    C = torch.full((i.tokens, i.ctx_width), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((i.tokens, i.q_heads), float("nan"), dtype=torch.float32, device="cuda")
    dQKV = torch.full((i.tokens, i.qkv_width), float("nan"), dtype=torch.bfloat16, device="cuda")
    q = G.dev(QKV)
    plan.attn_core_fwd(q, C, seq_len, lse=lse)
    plan.attn_core_bwd(q, C, lse, G.dev(dC), dQKV, seq_len)
    torch.cuda.synchronize()
    plan.close()
    return C, lse, dQKV


def _check_dqkv(dQKV, ref, qh, kvh, label=""):
    """Parity of dQ, dK and dV (each a tensor of its own) with the oracle."""
    q0, k0 = qh * 128, (qh + kvh) * 128
    G.assert_parity(dQKV[:, :q0], ref[:, :q0], "dQ" + label)
    G.assert_parity(dQKV[:, q0:k0], ref[:, q0:k0], "dK" + label)
    G.assert_parity(dQKV[:, k0:], ref[:, k0:], "dV" + label)


@pytest.mark.parametrize("tokens,seq_len,heads,kv_heads,tp", SMALL)
def test_attention_core_backward_small(tokens, seq_len, heads, kv_heads, tp):
    """dQ, dK and dV against the oracle's gradient (several key and query blocks per sequence,
    several sequences, grouped and ungrouped key/value heads); the forward's row log-sum-exp against
    the oracle's; the same bits on a second run; a sequence alone gives its rows of the batch."""
    w = synth.custom("attn_bwd", 940, tokens=tokens, hidden=256, ffn=64, tp=tp, act="gelu", bias=False,
                     row_slices=1, col_slices=1, heads=heads, kv_heads=kv_heads, head_dim=128)
    qh, kvh = w.q_heads_shard, w.kv_heads_shard
    _case("backward", tokens=tokens, seq_len=seq_len, q=qh, kv=kvh)
    QKV = synth.randn_bf16((tokens, w.qkv_width), 1.0, 941)
    dC = synth.randn_bf16((tokens, w.ctx_width), 1.0, 942)
    C, lse, dQKV = _run_bwd(w, QKV, dC, seq_len)
    f = L.as_f64
    ref_lse = A.attn_core_lse(f(QKV), qh, kvh, 128, seq_len)
    G.assert_parity(lse, ref_lse, "lse")
    ref = A.attn_core_bwd(f(QKV), f(dC), qh, kvh, 128, seq_len)
    _check_dqkv(dQKV, ref, qh, kvh)
    _, _, again = _run_bwd(w, QKV, dC, seq_len)
    assert torch.equal(again, dQKV)
    if tokens // seq_len > 1:
        w1 = synth.custom("attn_bwd1", 940, tokens=seq_len, hidden=256, ffn=64, tp=tp, act="gelu", bias=False,
                          row_slices=1, col_slices=1, heads=heads, kv_heads=kv_heads, head_dim=128)
        _, _, one = _run_bwd(w1, QKV[-seq_len:].contiguous(), dC[-seq_len:].contiguous(), seq_len)
        assert torch.equal(one, dQKV[-seq_len:])


def test_attention_core_backward_closed_forms():
    """Zero upstream gradient: dQKV is zero exactly. Zero values: dQ = dK = 0 exactly (dP = 0)."""
    w = synth.custom("attn_bwd_cf", 943, tokens=256, hidden=256, ffn=64, tp=2, act="gelu", bias=False,
                     row_slices=1, col_slices=1, heads=8, kv_heads=2, head_dim=128)
    qh, kvh = w.q_heads_shard, w.kv_heads_shard
    QKV = synth.randn_bf16((256, w.qkv_width), 1.0, 944)
    dC = synth.randn_bf16((256, w.ctx_width), 1.0, 945)
    _, _, d0 = _run_bwd(w, QKV, torch.zeros_like(dC), 128)
    assert torch.count_nonzero(d0.float()) == 0
    Z = QKV.clone()
    Z[:, (qh + kvh) * 128:] = 0
    _, _, dz = _run_bwd(w, Z, dC, 128)
    assert torch.count_nonzero(dz[:, :(qh + kvh) * 128].float()) == 0
    ref = A.attn_core_bwd(L.as_f64(Z), L.as_f64(dC), qh, kvh, 128, 128)
    G.assert_parity(dz[:, (qh + kvh) * 128:], ref[:, (qh + kvh) * 128:], "dV (zero values)")


@pytest.mark.parametrize("key", ["llama2_13b_layer", "llama3_70b_layer"])
def test_attention_core_backward_workload_sequence(key):
    """The workload's shard shape at 2048-token sequences: every row of the first and the last
    sequence against the oracle (sequences are independent)."""
    w = synth.WORKLOADS[key]
    seq = 2048
    qh, kvh = w.q_heads_shard, w.kv_heads_shard
    _case("backward workload", key=key, tokens=w.tokens, seq_len=seq)
    QKV = synth.randn_bf16((w.tokens, w.qkv_width), 1.0, 946)
    dC = synth.randn_bf16((w.tokens, w.ctx_width), 1.0, 947)
    _, _, dQKV = _run_bwd(w, QKV, dC, seq)
    f = L.as_f64
    for rows, label in ((slice(0, seq), " (first sequence)"), (slice(w.tokens - seq, w.tokens), " (last sequence)")):
        ref = A.attn_core_bwd(f(QKV[rows]), f(dC[rows]), qh, kvh, 128, seq)
        _check_dqkv(dQKV[rows], ref, qh, kvh, label)
