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


def _ramped_qkv(w, seq, seed):
    """QKV whose scores (log2 units, scale 1/sqrt(128) log2 e) follow a chosen level per 128-key block
    of each sequence: every query is 8 e1 and every key a_b e1 plus small noise, so a query's score
    against a key of block b is about 1.02 a_b. The levels make the row maximum stay within 2^8 of
    the first block's (a_1 = 5), jump past it (a_2 = 20), fall (a_3 = -10), rise to just under 2^8
    above the reference (a_4 = 27) and past it (a_5 = 29), then return near 0."""
    qh, kvh = w.q_heads_shard, w.kv_heads_shard
    g = torch.Generator().manual_seed(seed)
    QKV = (0.1 * torch.randn((w.tokens, w.qkv_width), generator=g)).float()
    levels = [0.0, 5.0, 20.0, -10.0, 27.0, 29.0] + [0.0] * 10
    pos = torch.arange(w.tokens) % seq
    a = torch.tensor([levels[p // 128] for p in pos.tolist()]) + 0.25 * torch.randn(w.tokens, generator=g)
    for h in range(qh):
        QKV[:, h * 128] = 8.0
    for k in range(kvh):
        QKV[:, (qh + k) * 128] = a
    return QKV.to(torch.bfloat16)


def _dq_large_key_bound(Q, K, V, dO, scale, qh):
    """Element bound on dQ[t, h, 0] (the dimension that carries the large keys) from the arithmetic
    of the backward: dQ = scale * sum_s dS[t, s] K[s] with dS = P (dP - D) rounded to bf16 (relative
    2^-9 each, taken as 2^-8), D = sum_d dO O computed from the forward's bf16 O (absolute error at
    most 2^-8 sum_d |dO O|, which enters every dS of the row times P), and dQ itself rounded to bf16.
    Since sum_s dS = 0, dQ along a direction where every key is large is a cancelling sum: its error
    follows sum_s |dS| |K|, not |dQ|. fp64, causal, one key/value head."""
    n = Q.shape[0]
    mask = np.tril(np.ones((n, n), dtype=bool))
    k0 = np.abs(K[:, 0])
    out = np.zeros((n, qh))
    for h in range(qh):
        q = Q[:, h * 128:(h + 1) * 128]
        S = np.where(mask, (q @ K.T) * scale, -np.inf)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        do = dO[:, h * 128:(h + 1) * 128]
        O = P @ V
        dP = do @ V.T
        D = (do * O).sum(axis=1, keepdims=True)
        dS = P * (dP - D)
        dq0 = scale * (dS @ K[:, 0])
        d_err = 2.0 ** -8 * np.abs(do * O).sum(axis=1)
        out[:, h] = 2.0 ** -8 * (scale * (np.abs(dS) @ k0) + np.abs(dq0)) + scale * d_err * (P @ k0) + 1e-6
    return out


def test_attention_core_moving_row_maximum():
    """Scores whose row maximum rises by less than 2^8 (the row keeps its softmax reference, P up to
    about 2^7) and by more (the reference moves), at the 70B shard shape (the four-wave forward
    kernel): the forward, the row log-sum-exp and the backward of the last sequence against the
    oracle, and that sequence alone (the eight-wave forward and dQ kernels) bit-equal to its rows of
    the batch (the four-wave ones).
    dQ along the large keys' dimension is checked against the bound of _dq_large_key_bound (the
    library before the lazy reference missed the plain Frobenius bound there by the same amount,
    4.6e-2 against 5e-3: bf16 dS times keys of 20-30)."""
    w = synth.WORKLOADS["llama3_70b_layer"]
    seq = 2048
    qh, kvh = w.q_heads_shard, w.kv_heads_shard
    _case("moving maximum", key=w.key, tokens=w.tokens, seq_len=seq)
    QKV = _ramped_qkv(w, seq, 950)
    dC = synth.randn_bf16((w.tokens, w.ctx_width), 1.0, 951)
    C, lse, dQKV = _run_bwd(w, QKV, dC, seq)
    f = L.as_f64
    last = slice(w.tokens - seq, w.tokens)
    G.assert_parity(C[last], A.attn_core_fwd(f(QKV[last]), qh, kvh, 128, seq), "C (last sequence)")
    G.assert_parity(lse[last], A.attn_core_lse(f(QKV[last]), qh, kvh, 128, seq), "lse (last sequence)")
    ref = A.attn_core_bwd(f(QKV[last]), f(dC[last]), qh, kvh, 128, seq)
    q0, k0 = qh * 128, (qh + kvh) * 128
    G.assert_parity(dQKV[last][:, q0:k0], ref[:, q0:k0], "dK (last sequence)")
    G.assert_parity(dQKV[last][:, k0:], ref[:, k0:], "dV (last sequence)")
    other = [c for c in range(q0) if c % 128 != 0]
    G.assert_parity(dQKV[last][:, other], ref[:, other], "dQ except the large keys' dimension")
    Qf, Kf, Vf = f(QKV[last])[:, :q0], f(QKV[last])[:, q0:k0], f(QKV[last])[:, k0:]
    bound = _dq_large_key_bound(Qf, Kf, Vf, f(dC[last]), 1.0 / np.sqrt(128.0), qh)
    err = np.abs(dQKV[last][:, 0:q0:128].float().cpu().numpy() - ref[:, 0:q0:128])
    worst = float((err / bound).max())
    print(f"dQ along the large keys: max error / bound {worst:.3f}", flush=True)
    assert worst <= 1.0
    w1 = synth.custom("attn_move1", 952, tokens=seq, hidden=8192, ffn=64, tp=8, act="swiglu", bias=False,
                      row_slices=1, col_slices=1, heads=64, kv_heads=8, head_dim=128)
    assert (w1.q_heads_shard, w1.kv_heads_shard) == (qh, kvh)
    C1, lse1, dQKV1 = _run_bwd(w1, QKV[last].contiguous(), dC[last].contiguous(), seq)
    assert torch.equal(C1, C[last])
    assert torch.equal(lse1, lse[last])
    # the batch's dQ comes from the four-wave dQ kernel (1024 blocks), the sequence's from the
    # eight-wave one (64 blocks)
    assert torch.equal(dQKV1, dQKV[last])
