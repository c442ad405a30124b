"""Pins of the fp64 oracle (CPU only), and planted mistakes that the pins must catch."""
import copy
import math
import types

import numpy as np
import pytest

from oracle import layer as L
from oracle import plan as P
from oracle.compare import compare
import pins


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
@pytest.mark.parametrize("bias", [True, False])
@pytest.mark.parametrize("seed", [0, 7])
def test_brute_force_mlp(act, bias, seed):
    pins.check_brute_mlp(L, act, seed=seed, bias=bias)


@pytest.mark.parametrize("bias", [True, False])
def test_brute_force_attnproj(bias):
    pins.check_brute_attnproj(L, bias=bias)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
@pytest.mark.parametrize("bias", [True, False])
def test_finite_difference_mlp(act, bias):
    pins.check_fd_mlp(L, act, bias=bias, seed=3)


def test_finite_difference_attnproj():
    pins.check_fd_attnproj(L, seed=5)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_torch_autograd_float64(act):
    pins.check_torch_mlp(L, act, bias=(act == "gelu"))


def test_textbook_values():
    pins.check_textbook(L)


def test_activation_special_values():
    pins.check_activation_limits(L)


def test_library_activations():
    pins.check_library_activations(L)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_tp_sum_invariance(act):
    pins.check_tp_sum(L, act, bias=(act == "gelu"))


def test_tp_sum_invariance_tiny_workload_shape():
    """The tiny GPT workload: h=512, F=2048 at TP 1/4 (shard 512), with a row-parallel bias."""
    pins.check_tp_sum(L, "gelu", tp=4, M=8, h=512, F=2048, bias=True)


# ------------------------------------------------------------------------------- closed forms
def test_closed_forms():
    rng = np.random.default_rng(1)
    M, h = 6, 8
    X = rng.standard_normal((M, h))
    W1 = rng.standard_normal((h, h))
    b1 = rng.standard_normal(h)
    W2 = rng.standard_normal((h, h))
    # W2 = 0  =>  Z = 0 exactly
    assert np.all(L.mlp_fwd(X, W1, b1, np.zeros_like(W2), "gelu")["Z"] == 0.0)
    # W1 = 0  =>  every row of Z equals act(b1) W2^T
    Z = L.mlp_fwd(X, np.zeros_like(W1), b1, W2, "gelu")["Z"]
    row = (0.5 * b1 * (1 + np.vectorize(__import__("math").erf)(b1 / np.sqrt(2)))) @ W2.T
    assert np.allclose(Z, np.broadcast_to(row, Z.shape), rtol=1e-14, atol=1e-14)
    # identity weights: Z = gelu(X) ; SwiGLU with W_g = W_u = I: Z = silu(X) X
    I = np.eye(h)
    from scipy.special import ndtr
    assert np.allclose(L.mlp_fwd(X, I, None, I, "gelu")["Z"], X * ndtr(X), rtol=1e-14, atol=1e-15)
    Zs = L.mlp_fwd(X, np.concatenate([I, I]), None, I, "swiglu")["Z"]
    assert np.allclose(Zs, X * X / (1 + np.exp(-X)), rtol=1e-14, atol=1e-15)
    # gate and up are distinguished: W_g = I, W_u = 2 I gives 2 silu(X) X, not silu(2X) X
    Zg = L.mlp_fwd(X, np.concatenate([I, 2 * I]), None, I, "swiglu")["Z"]
    assert np.allclose(Zg, 2 * X * X / (1 + np.exp(-X)), rtol=1e-14, atol=1e-15)


def test_attnproj_closed_forms():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((5, 4))
    C = rng.standard_normal((5, 3))
    o = L.attnproj_fwd(X, np.eye(4), None, C, np.zeros((4, 3)))
    assert np.array_equal(o["QKV"], X) and np.all(o["Z"] == 0)


# ------------------------------------------------------------------------------- slice geometry
def test_even_ranges_cover_and_order():
    for n, p in [(256, 2), (8192, 4), (16384, 8), (2560, 2), (4096, 2), (7, 7), (12, 1)]:
        rs = P.even_ranges(n, p)
        assert rs[0][0] == 0 and rs[-1][1] == n and len(rs) == p
        assert all(rs[i][1] == rs[i + 1][0] for i in range(p - 1))
        assert len({b - a for a, b in rs}) == 1
    for n, p in [(10, 3), (0, 1), (5, 0)]:
        with pytest.raises(ValueError):
            P.even_ranges(n, p)


def test_handoff_pieces_tile_exactly_once():
    for rows, cols, r, c in [(256, 512, 2, 2), (16384, 8192, 8, 2), (24, 40, 3, 5)]:
        cover = np.zeros((rows, cols), dtype=np.int32)
        pieces = P.handoff_pieces(rows, cols, r, c)
        assert len(pieces) == r * c
        for (a, b, x, y) in pieces:
            cover[a:b, x:y] += 1
        assert np.all(cover == 1)
        assert pieces == sorted(pieces)  # row slice major, ascending


# ----------------------------------------------------------------------------------- comparator
def test_comparator_accepts_and_rejects():
    rng = np.random.default_rng(4)
    o = rng.standard_normal((64, 48))
    assert compare(o, o).ok
    # bf16-level rounding noise passes
    g = o * (1 + rng.uniform(-2 ** -9, 2 ** -9, o.shape))
    assert compare(g, o).ok
    # one large elementwise error fails the elementwise test
    g = o.copy(); g[3, 5] += 0.5
    v = compare(g, o)
    assert not v.ok and v.n_elem_violations == 1 and v.worst_index == (3, 5)
    # 1% relative noise everywhere fails the Frobenius test (elementwise bound alone would pass)
    g = o * (1 + 0.01 * rng.choice([-1, 1], o.shape))
    v = compare(g, o)
    assert not v.ok and v.n_elem_violations == 0 and v.rel_fro > 5e-3
    g = o.copy(); g[0, 0] = np.nan
    assert not compare(g, o).ok
    with pytest.raises(ValueError):
        compare(o[:, :3], o)


# ------------------------------------------------------------------------------ planted mistakes
def _mutant(**overrides):
    """A copy of the oracle's layer module with some functions replaced."""
    m = types.ModuleType("oracle_mutant")
    m.__dict__.update({k: v for k, v in vars(L).items() if not k.startswith("__")})
    m.__dict__.update(overrides)
    # module functions look up globals in their own module: rebind them to the mutant namespace
    for k, v in list(m.__dict__.items()):
        if isinstance(v, types.FunctionType) and k not in overrides:
            m.__dict__[k] = types.FunctionType(v.__code__, m.__dict__, k, v.__defaults__, v.__closure__)
    return m


def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_planted_gelu_prime_missing_density_term():
    bad = _mutant(gelu_prime=lambda u: 0.5 * (1.0 + L.erf(u * L._INV_SQRT2)))
    assert _fails(lambda: pins.check_fd_mlp(bad, "gelu"))


def test_planted_silu_prime_wrong_sign():
    def silu_prime(g):
        s = L.sigmoid(g)
        return s * (1.0 - g * (1.0 - s))
    bad = _mutant(silu_prime=silu_prime)
    assert _fails(lambda: pins.check_fd_mlp(bad, "swiglu"))


def test_planted_gate_up_swapped():
    def activate(U, act):
        if act == "swiglu":
            G, V = L._split_gate_up(U)
            return L.silu(V) * G
        return L.gelu(U)
    bad = _mutant(activate=activate)
    assert _fails(lambda: pins.check_brute_mlp(bad, "swiglu"))


def test_planted_bias_dropped():
    def mlp_fwd(X, W1, b1, W2, act):
        U = X @ W1.T
        H = L.activate(U, act)
        return {"U": U, "H": H, "Z": H @ W2.T}
    bad = _mutant(mlp_fwd=mlp_fwd)
    assert _fails(lambda: pins.check_brute_mlp(bad, "gelu", bias=True))


def test_planted_transposed_operand_in_dgrad():
    def mlp_bwd(X, W1, W2, U, dY, act, with_bias=False):
        out = L.mlp_bwd(X, W1, W2, U, dY, act, with_bias)
        out["dW2"] = out["dW2"][::-1]  # rows in the wrong order
        return out
    bad = _mutant(mlp_bwd=mlp_bwd)
    assert _fails(lambda: pins.check_fd_mlp(bad, "gelu"))


def test_planted_gelu_tanh_form_instead_of_erf():
    def gelu(u):
        return 0.5 * u * (1 + np.tanh(np.sqrt(2 / np.pi) * (u + 0.044715 * u ** 3)))
    bad = _mutant(gelu=gelu)
    assert _fails(lambda: pins.check_textbook(bad))


def test_planted_row_parallel_bias_added_to_every_partial():
    def mlp_fwd(X, W1, b1, W2, act):
        o = L.mlp_fwd(X, W1, b1, W2, act)
        o["Z"] = o["Z"] + 0.05  # a bias folded into each partial sum
        return o
    bad = _mutant(mlp_fwd=mlp_fwd)
    assert _fails(lambda: pins.check_tp_sum(bad, "gelu"))


# ---------------------------------------------------------------- attention core (causal, GQA)
from oracle import attention as A  # noqa: E402


def _brute_attn(QKV, qh, kvh, d, S):
    """Triple loop with math.exp: the definition on tiny shapes."""
    M = len(QKV)
    out = [[0.0] * (qh * d) for _ in range(M)]
    for b in range(M // S):
        for h in range(qh):
            g = h // (qh // kvh)
            for t in range(S):
                T = b * S + t
                sc = []
                for s_ in range(t + 1):
                    Ss = b * S + s_
                    sc.append(sum(QKV[T][h * d + i] * QKV[Ss][(qh + g) * d + i] for i in range(d)) / math.sqrt(d))
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                z = sum(w)
                for i in range(d):
                    out[T][h * d + i] = sum(w[j] * QKV[b * S + j][(qh + kvh + g) * d + i] for j in range(t + 1)) / z
    return np.array(out)


def test_attention_brute_force():
    rng = np.random.default_rng(3)
    for qh, kvh, d, S, nb in [(2, 1, 3, 5, 2), (4, 2, 4, 4, 1), (3, 3, 2, 6, 1)]:
        QKV = rng.standard_normal((S * nb, (qh + 2 * kvh) * d))
        got = A.attn_core_fwd(QKV, qh, kvh, d, S)
        ref = _brute_attn(QKV.tolist(), qh, kvh, d, S)
        assert np.max(np.abs(got - ref)) < 1e-12


def test_attention_closed_forms():
    rng = np.random.default_rng(4)
    qh, kvh, d, S = 4, 2, 8, 16
    QKV = rng.standard_normal((2 * S, (qh + 2 * kvh) * d))
    q, k, v = A.split_qkv(QKV, qh, kvh, d)
    C = A.attn_core_fwd(QKV, qh, kvh, d, S).reshape(2 * S, qh, d)
    # the first token of each sequence sees only itself: C = its own V, exactly
    for b in range(2):
        for h in range(qh):
            assert np.array_equal(C[b * S, h], v[b * S, h // 2])
    # zero keys: uniform weights, C[t] = mean of V[0..t] of the sequence
    Z = QKV.copy()
    Z[:, qh * d:(qh + kvh) * d] = 0.0
    Cz = A.attn_core_fwd(Z, qh, kvh, d, S).reshape(2 * S, qh, d)
    for t in range(S):
        np.testing.assert_allclose(Cz[S + t, 1], v[S:S + t + 1, 0].mean(axis=0), rtol=0, atol=1e-13)
    # a constant vector added to every key of a head shifts a row's scores by one amount: no change
    Sh = QKV.copy()
    Sh[:, qh * d:(qh + 1) * d] += rng.standard_normal(d)
    np.testing.assert_allclose(A.attn_core_fwd(Sh, qh, kvh, d, S), A.attn_core_fwd(QKV, qh, kvh, d, S),
                               rtol=0, atol=1e-12)
    # query heads of one group with the same queries give the same outputs (grouped KV heads)
    G = QKV.copy()
    G[:, d:2 * d] = G[:, 0:d]
    Cg = A.attn_core_fwd(G, qh, kvh, d, S).reshape(2 * S, qh, d)
    assert np.array_equal(Cg[:, 0], Cg[:, 1])
    # sequences are independent: each sequence alone gives the same rows
    np.testing.assert_array_equal(A.attn_core_fwd(QKV[S:], qh, kvh, d, S), A.attn_core_fwd(QKV, qh, kvh, d, S)[S:])


def test_attention_backward_finite_differences():
    for qh, kvh, d, S, nb in [(4, 2, 3, 4, 2), (2, 1, 4, 5, 1), (3, 3, 2, 3, 2)]:
        pins.check_fd_attn_core(A, seed=qh + d, qh=qh, kvh=kvh, d=d, S=S, nb=nb)


def test_attention_backward_torch_autograd():
    pins.check_torch_attn_core(A, qh=4, kvh=1)
    pins.check_torch_attn_core(A, seed=1, qh=4, kvh=2, d=8, S=7, nb=3)


def test_attention_lse():
    pins.check_lse(A)
    pins.check_lse(A, seed=2, qh=4, kvh=2)


def test_attention_backward_closed_forms():
    rng = np.random.default_rng(6)
    qh, kvh, d, S = 4, 2, 6, 8
    QKV = rng.standard_normal((2 * S, (qh + 2 * kvh) * d))
    dC = rng.standard_normal((2 * S, qh * d))
    # zero upstream gradient: zero everywhere, exactly
    assert not np.any(A.attn_core_bwd(QKV, np.zeros_like(dC), qh, kvh, d, S))
    # zero values: dP = 0, so dQ = dK = 0 exactly; dV[s] = sum over the group's heads and t >= s of P[t, s] dC[t]
    Z = QKV.copy()
    Z[:, (qh + kvh) * d:] = 0.0
    g = A.attn_core_bwd(Z, dC, qh, kvh, d, S)
    assert not np.any(g[:, :(qh + kvh) * d])
    # the last token of a sequence is seen only by itself: its dV is P[last, last] dC[last] summed over heads
    q, k, _ = A.split_qkv(Z, qh, kvh, d)
    lse = A.attn_core_lse(Z, qh, kvh, d, S)
    last = S - 1
    for gi in range(kvh):
        ref = sum(np.exp(q[last, h] @ k[last, gi] / np.sqrt(d) - lse[last, h]) * dC[last, h * d:(h + 1) * d]
                  for h in range(gi * 2, gi * 2 + 2))
        np.testing.assert_allclose(g[last, (qh + kvh + gi) * d:(qh + kvh + gi + 1) * d], ref, rtol=1e-13, atol=1e-14)
    # sequences are independent
    np.testing.assert_array_equal(A.attn_core_bwd(QKV[S:], dC[S:], qh, kvh, d, S),
                                  A.attn_core_bwd(QKV, dC, qh, kvh, d, S)[S:])


def _mutant_attn(**overrides):
    m = types.ModuleType("attention_mutant")
    m.__dict__.update(A.__dict__)
    m.__dict__.update(overrides)
    return m


def test_planted_attention_dk_dv_swapped():
    def attn_core_bwd(QKV, dC, qh, kvh, d, S):
        g = A.attn_core_bwd(QKV, dC, qh, kvh, d, S)
        k0, v0 = qh * d, (qh + kvh) * d
        return np.concatenate([g[:, :k0], g[:, v0:], g[:, k0:v0]], axis=1)
    assert _fails(lambda: pins.check_fd_attn_core(_mutant_attn(attn_core_bwd=attn_core_bwd)))


def test_planted_attention_dq_scale_missing():
    def attn_core_bwd(QKV, dC, qh, kvh, d, S):
        g = A.attn_core_bwd(QKV, dC, qh, kvh, d, S).copy()
        g[:, :qh * d] *= np.sqrt(d)
        return g
    assert _fails(lambda: pins.check_fd_attn_core(_mutant_attn(attn_core_bwd=attn_core_bwd)))


def test_planted_attention_gqa_gradient_not_summed():
    def attn_core_bwd(QKV, dC, qh, kvh, d, S):
        # each key/value head keeps only its last query head's share (assignment instead of a sum)
        g = A.attn_core_bwd(QKV, dC, qh, kvh, d, S).copy()
        keep = dC.copy()
        grp = qh // kvh
        for h in range(qh):
            if h % grp != grp - 1:
                keep[:, h * d:(h + 1) * d] = 0.0
        part = A.attn_core_bwd(QKV, keep, qh, kvh, d, S)
        g[:, qh * d:] = part[:, qh * d:]
        return g
    assert _fails(lambda: pins.check_fd_attn_core(_mutant_attn(attn_core_bwd=attn_core_bwd)))
