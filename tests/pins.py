"""Independent checks that pin the fp64 oracle to things other than itself.

Each check takes the oracle module as an argument so that the planted-mistake tests can hand it a
copy with one deliberate error and show that some check fails.

  brute_*      exact rational arithmetic (fractions.Fraction) on the bf16 inputs for every linear part,
               scalar math.erf / math.exp for the activations; loops only, tiny shapes.
  fd_*         central finite differences of L = <dY, output> through the oracle's forward.
  torch_*      torch.autograd in float64 with torch's own GELU/SiLU: an independent library.
  textbook     standard-normal CDF and logistic values from tests/golden/.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def bf16_array(shape, std, seed, dtype=np.float64):
    """Small random arrays whose entries are bf16-representable (so Fraction(x) is exact)."""
    g = torch.Generator().manual_seed(seed)
    t = (torch.randn(*shape, generator=g) * std).to(torch.bfloat16).float()
    return t.numpy().astype(dtype)


# --------------------------------------------------------------------------------- brute force
def _gelu_s(u: float) -> float:
    return u * 0.5 * (1.0 + math.erf(u / math.sqrt(2.0)))


def _silu_s(g: float) -> float:
    return g / (1.0 + math.exp(-g)) if g >= 0 else g * math.exp(g) / (1.0 + math.exp(g))


def brute_mlp_fwd(X, W1, b1, W2, act):
    """Loops: U[m][n] = sum_k X[m][k] W1[n][k] (+ b1[n]) exactly; H by scalar activation;
    Z[m][j] = sum_f H[m][f] W2[j][f] exactly in rationals of the fp64 H."""
    M, h = X.shape
    N1 = W1.shape[0]
    Fp = W2.shape[1]
    U = [[sum(Fraction(float(X[m, k])) * Fraction(float(W1[n, k])) for k in range(h))
          + (Fraction(float(b1[n])) if b1 is not None else 0) for n in range(N1)] for m in range(M)]
    H = [[0.0] * Fp for _ in range(M)]
    for m in range(M):
        for f in range(Fp):
            if act == "gelu":
                H[m][f] = _gelu_s(float(U[m][f]))
            else:
                H[m][f] = _silu_s(float(U[m][f])) * float(U[m][Fp + f])
    Z = [[float(sum(Fraction(H[m][f]) * Fraction(float(W2[j, f])) for f in range(Fp)))
          for j in range(W2.shape[0])] for m in range(M)]
    return np.array([[float(x) for x in row] for row in U]), np.array(H), np.array(Z)


def brute_attnproj_fwd(X, Wqkv, bqkv, C, Wo):
    M, h = X.shape
    QKV = [[float(sum(Fraction(float(X[m, k])) * Fraction(float(Wqkv[n, k])) for k in range(h))
                  + (Fraction(float(bqkv[n])) if bqkv is not None else 0))
            for n in range(Wqkv.shape[0])] for m in range(M)]
    Z = [[float(sum(Fraction(float(C[m, k])) * Fraction(float(Wo[n, k])) for k in range(C.shape[1])))
          for n in range(Wo.shape[0])] for m in range(M)]
    return np.array(QKV), np.array(Z)


def assert_close(a, b, rtol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rtol * scale, f"{what}: max err {err:.3e} > {rtol:.1e} * {scale:.3e}"


def check_brute_mlp(oracle_layer, act, seed=0, M=5, h=6, Fp=4, bias=True):
    X = bf16_array((M, h), 1.0, seed + 1)
    N1 = 2 * Fp if act == "swiglu" else Fp
    W1 = bf16_array((N1, h), 0.5, seed + 2)
    b1 = bf16_array((N1,), 0.3, seed + 3) if bias else None
    W2 = bf16_array((h + 1, Fp), 0.5, seed + 4)  # output width != input width: catches transposes
    U, H, Z = brute_mlp_fwd(X, W1, b1, W2, act)
    o = oracle_layer.mlp_fwd(X, W1, b1, W2, act)
    assert_close(o["U"], U, 1e-14, "U")
    assert_close(o["H"], H, 1e-14, "H")
    assert_close(o["Z"], Z, 1e-14, "Z")


def check_brute_attnproj(oracle_layer, seed=0, M=4, h=6, nqkv=5, ctx=3, bias=True):
    X = bf16_array((M, h), 1.0, seed + 1)
    Wqkv = bf16_array((nqkv, h), 0.5, seed + 2)
    bqkv = bf16_array((nqkv,), 0.3, seed + 3) if bias else None
    C = bf16_array((M, ctx), 1.0, seed + 4)
    Wo = bf16_array((h, ctx), 0.5, seed + 5)
    QKV, Z = brute_attnproj_fwd(X, Wqkv, bqkv, C, Wo)
    o = oracle_layer.attnproj_fwd(X, Wqkv, bqkv, C, Wo)
    assert_close(o["QKV"], QKV, 1e-14, "QKV")
    assert_close(o["Z"], Z, 1e-14, "Z")


# ---------------------------------------------------------------------------- finite differences
def _fd(fun, x, idx, eps=1e-6):
    xp = x.copy(); xp[idx] += eps
    xm = x.copy(); xm[idx] -= eps
    return (fun(xp) - fun(xm)) / (2 * eps)


def check_fd_mlp(oracle_layer, act, seed=0, M=4, h=5, Fp=3, bias=True, n_probe=6):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, h))
    N1 = 2 * Fp if act == "swiglu" else Fp
    W1 = rng.standard_normal((N1, h)) * 0.7
    b1 = rng.standard_normal(N1) * 0.3 if bias else None
    W2 = rng.standard_normal((h + 2, Fp)) * 0.7
    dY = rng.standard_normal((M, h + 2))
    U = X @ W1.T + (b1 if bias else 0.0)
    g = oracle_layer.mlp_bwd(X, W1, W2, U, dY, act, with_bias=bias)

    def L(X_=X, W1_=W1, b1_=b1, W2_=W2):
        return float(np.sum(dY * oracle_layer.mlp_fwd(X_, W1_, b1_, W2_, act)["Z"]))

    params = [("dX", X, lambda v: L(X_=v)), ("dW1", W1, lambda v: L(W1_=v)),
              ("dW2", W2, lambda v: L(W2_=v))]
    if bias:
        params.append(("db1", b1, lambda v: L(b1_=v)))
    for name, arr, fun in params:
        for _ in range(n_probe):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            fd = _fd(fun, arr, idx)
            an = g[name][idx]
            assert abs(fd - an) <= 1e-6 * (1 + abs(fd)), f"{act} {name}{idx}: fd {fd} vs {an}"


def check_fd_attnproj(oracle_layer, seed=0, M=3, h=4, nqkv=5, ctx=3, n_probe=6):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, h))
    Wqkv = rng.standard_normal((nqkv, h))
    bqkv = rng.standard_normal(nqkv)
    C = rng.standard_normal((M, ctx))
    Wo = rng.standard_normal((h, ctx))
    dQKV = rng.standard_normal((M, nqkv))
    dY = rng.standard_normal((M, h))
    g = oracle_layer.attnproj_bwd(X, Wqkv, dQKV, C, Wo, dY, with_bias=True)

    def L(X_=X, Wqkv_=Wqkv, bqkv_=bqkv, C_=C, Wo_=Wo):
        o = oracle_layer.attnproj_fwd(X_, Wqkv_, bqkv_, C_, Wo_)
        return float(np.sum(dQKV * o["QKV"]) + np.sum(dY * o["Z"]))

    params = [("dX", X, lambda v: L(X_=v)), ("dWqkv", Wqkv, lambda v: L(Wqkv_=v)),
              ("dbqkv", bqkv, lambda v: L(bqkv_=v)), ("dC", C, lambda v: L(C_=v)),
              ("dWo", Wo, lambda v: L(Wo_=v))]
    for name, arr, fun in params:
        for _ in range(n_probe):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            fd = _fd(fun, arr, idx)
            an = g[name][idx]
            assert abs(fd - an) <= 1e-6 * (1 + abs(fd)), f"attn {name}{idx}: fd {fd} vs {an}"


# ------------------------------------------------------------------------------- torch autograd
def check_torch_mlp(oracle_layer, act, seed=0, M=6, h=8, Fp=5, bias=True):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, h))
    N1 = 2 * Fp if act == "swiglu" else Fp
    W1 = rng.standard_normal((N1, h)) * 0.5
    b1 = rng.standard_normal(N1) * 0.2 if bias else None
    W2 = rng.standard_normal((h, Fp)) * 0.5
    dY = rng.standard_normal((M, h))
    tX, tW1, tW2 = (torch.tensor(a, requires_grad=True) for a in (X, W1, W2))
    tb1 = torch.tensor(b1, requires_grad=True) if bias else None
    U = torch.nn.functional.linear(tX, tW1, tb1)
    if act == "gelu":
        H = torch.nn.functional.gelu(U)
    else:
        H = torch.nn.functional.silu(U[:, :Fp]) * U[:, Fp:]
    Z = torch.nn.functional.linear(H, tW2)
    Z.backward(torch.tensor(dY))
    o = oracle_layer.mlp_fwd(X, W1, b1, W2, act)
    assert_close(o["Z"], Z.detach().numpy(), 1e-13, "torch Z")
    g = oracle_layer.mlp_bwd(X, W1, W2, U.detach().numpy(), dY, act, with_bias=bias)
    assert_close(g["dX"], tX.grad.numpy(), 1e-13, "torch dX")
    assert_close(g["dW1"], tW1.grad.numpy(), 1e-13, "torch dW1")
    assert_close(g["dW2"], tW2.grad.numpy(), 1e-13, "torch dW2")
    if bias:
        assert_close(g["db1"], tb1.grad.numpy(), 1e-13, "torch db1")


# ------------------------------------------------------------------------------ textbook values
def load_textbook():
    rows = []
    with open(os.path.join(GOLDEN, "normal_cdf_logistic.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, x, v = line.split()
            rows.append((kind, float(x), float(v)))
    return rows


def check_textbook(oracle_layer):
    for kind, x, v in load_textbook():
        xa = np.array([x])
        if kind == "Phi":
            # gelu(x) = x Phi(x); at x = 0 use the derivative gelu'(0) = Phi(0)
            if x == 0.0:
                got = float(oracle_layer.gelu_prime(xa)[0])
            else:
                got = float(oracle_layer.gelu(xa)[0]) / x
        else:
            got = float(oracle_layer.sigmoid(xa)[0])
            if x != 0.0:
                assert abs(float(oracle_layer.silu(xa)[0]) - x * v) <= 1e-15 * (1 + abs(x)), \
                    f"silu({x})"
        assert abs(got - v) <= 2e-15, f"{kind}({x}) = {got!r}, table {v!r}"


def check_activation_limits(oracle_layer):
    u = np.array([0.0])
    assert oracle_layer.gelu(u)[0] == 0.0
    assert abs(oracle_layer.gelu_prime(u)[0] - 0.5) < 1e-16
    assert oracle_layer.silu(u)[0] == 0.0
    assert abs(oracle_layer.silu_prime(u)[0] - 0.5) < 1e-16
    big = np.array([40.0, -40.0])
    assert abs(oracle_layer.gelu(big)[0] - 40.0) < 1e-12 and abs(oracle_layer.gelu(big)[1]) < 1e-12
    assert abs(oracle_layer.gelu_prime(big)[0] - 1.0) < 1e-12 and abs(oracle_layer.gelu_prime(big)[1]) < 1e-12
    huge = np.array([800.0, -800.0])
    s = oracle_layer.sigmoid(huge)
    assert s[0] == 1.0 and s[1] == 0.0 and np.all(np.isfinite(oracle_layer.silu(huge)))
    assert abs(oracle_layer.silu_prime(big)[0] - 1.0) < 1e-12 and abs(oracle_layer.silu_prime(big)[1]) < 1e-12


def check_library_activations(oracle_layer):
    """scipy's normal CDF (ndtr, a routine separate from erf) and torch's float64 GELU / SiLU."""
    from scipy.special import ndtr
    x = np.linspace(-6, 6, 97)
    assert np.max(np.abs(oracle_layer.gelu(x) - x * ndtr(x))) < 1e-14
    tx = torch.tensor(x)
    assert np.max(np.abs(oracle_layer.gelu(x) - torch.nn.functional.gelu(tx).numpy())) < 1e-14
    assert np.max(np.abs(oracle_layer.silu(x) - torch.nn.functional.silu(tx).numpy())) < 1e-14


# -------------------------------------------------------------------------- TP-sum invariance
def check_tp_sum(oracle_layer, act, tp=4, seed=0, M=16, h=32, F=64, bias=True):
    """Summing every rank's partial output (plus the row-parallel bias once) gives the unsharded
    layer, and each rank's weight gradients are the matching rows/columns of the unsharded ones."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, h))
    Fs = F // tp
    if act == "swiglu":
        Wg = rng.standard_normal((F, h)) * 0.1
        Wu = rng.standard_normal((F, h)) * 0.1
        W1_full = np.concatenate([Wg, Wu], axis=0)
    else:
        W1_full = rng.standard_normal((F, h)) * 0.1
    b1_full = rng.standard_normal(W1_full.shape[0]) * 0.1 if bias else None
    W2_full = rng.standard_normal((h, F)) * 0.1
    b2 = rng.standard_normal(h) * 0.1
    dY = rng.standard_normal((M, h))
    full = oracle_layer.mlp_fwd(X, W1_full, b1_full, W2_full, act)
    gfull = oracle_layer.mlp_bwd(X, W1_full, W2_full, full["U"], dY, act, with_bias=bias)
    acc = np.zeros((M, h))
    dX = np.zeros((M, h))
    for t in range(tp):
        cols = np.arange(t * Fs, (t + 1) * Fs)
        rows1 = np.concatenate([cols, F + cols]) if act == "swiglu" else cols
        W1 = W1_full[rows1]
        b1 = b1_full[rows1] if bias else None
        W2 = W2_full[:, cols]
        part = oracle_layer.mlp_fwd(X, W1, b1, W2, act)
        acc += part["Z"]
        g = oracle_layer.mlp_bwd(X, W1, W2, part["U"], dY, act, with_bias=bias)
        dX += g["dX"]
        assert_close(g["dW1"], gfull["dW1"][rows1], 1e-12, "dW1 shard")
        assert_close(g["dW2"], gfull["dW2"][:, cols], 1e-12, "dW2 shard")
        if bias:
            assert_close(g["db1"], gfull["db1"][rows1], 1e-12, "db1 shard")
    assert_close(acc + b2, full["Z"] + b2, 1e-12, "sum of partial Z")
    assert_close(dX, gfull["dX"], 1e-12, "sum of partial dX")
    # the unsharded reference written without the oracle's helpers
    U = X @ W1_full.T + (b1_full if bias else 0.0)
    if act == "gelu":
        from scipy.special import ndtr
        H = U * ndtr(U)
    else:
        H = U[:, :F] / (1.0 + np.exp(-U[:, :F])) * U[:, F:]
    assert_close(acc + b2, H @ W2_full.T + b2, 1e-12, "unsharded layer")


# ------------------------------------------------------------------- attention core, backward
def check_fd_attn_core(attn, seed=0, qh=4, kvh=2, d=3, S=4, nb=2, tol=1e-7):
    """Every entry of the oracle's dQKV against central differences of L = <dC, C(QKV)>, with C from
    the oracle's forward (itself pinned by a brute-force loop)."""
    rng = np.random.default_rng(seed)
    M = S * nb
    QKV = rng.standard_normal((M, (qh + 2 * kvh) * d))
    dC = rng.standard_normal((M, qh * d))
    g = attn.attn_core_bwd(QKV, dC, qh, kvh, d, S)
    assert g.shape == QKV.shape

    def L(v):
        return float(np.sum(dC * attn.attn_core_fwd(v, qh, kvh, d, S)))

    for idx in np.ndindex(*QKV.shape):
        fd = _fd(L, QKV, idx)
        assert abs(fd - g[idx]) <= tol * (1 + abs(fd)), f"dQKV{idx}: fd {fd} vs {g[idx]}"


def check_torch_attn_core(attn, seed=0, qh=4, kvh=1, d=5, S=6, nb=2):
    """The oracle's dQKV against torch autograd (fp64, CPU) through a torch statement of the
    forward pass: the gradient comes from the library's own differentiation."""
    import torch
    rng = np.random.default_rng(seed)
    M = S * nb
    QKV = rng.standard_normal((M, (qh + 2 * kvh) * d))
    dC = rng.standard_normal((M, qh * d))
    x = torch.tensor(QKV, dtype=torch.float64, requires_grad=True)
    q = x[:, :qh * d].reshape(nb, S, qh, d).permute(0, 2, 1, 3)
    k = x[:, qh * d:(qh + kvh) * d].reshape(nb, S, kvh, d).permute(0, 2, 1, 3)
    v = x[:, (qh + kvh) * d:].reshape(nb, S, kvh, d).permute(0, 2, 1, 3)
    k = k.repeat_interleave(qh // kvh, dim=1)
    v = v.repeat_interleave(qh // kvh, dim=1)
    sc = (q @ k.transpose(-1, -2)) / np.sqrt(d)
    mask = torch.ones(S, S, dtype=torch.bool).tril()
    sc = sc.masked_fill(~mask, float("-inf"))
    out = torch.softmax(sc, dim=-1) @ v                      # [nb][qh][S][d]
    out = out.permute(0, 2, 1, 3).reshape(M, qh * d)
    out.backward(torch.tensor(dC, dtype=torch.float64))
    got = attn.attn_core_bwd(QKV, dC, qh, kvh, d, S)
    assert_close(got, x.grad.numpy(), 1e-12, "dQKV (torch autograd)")


def check_lse(attn, seed=0, qh=3, kvh=1, d=4, S=5, nb=2):
    """Row log-sum-exp: a brute-force loop with math.exp / math.log, and the closed form log(t + 1)
    at zero keys (every score 0)."""
    rng = np.random.default_rng(seed)
    M = S * nb
    QKV = rng.standard_normal((M, (qh + 2 * kvh) * d))
    got = attn.attn_core_lse(QKV, qh, kvh, d, S)
    for b in range(nb):
        for h in range(qh):
            g = h // (qh // kvh)
            for t in range(S):
                T = b * S + t
                sc = [sum(QKV[T, h * d + i] * QKV[b * S + s, (qh + g) * d + i] for i in range(d)) / math.sqrt(d)
                      for s in range(t + 1)]
                ref = math.log(sum(math.exp(x) for x in sc))
                assert abs(got[T, h] - ref) <= 1e-12 * (1 + abs(ref)), (T, h, got[T, h], ref)
    Z = QKV.copy()
    Z[:, qh * d:(qh + kvh) * d] = 0.0
    z = attn.attn_core_lse(Z, qh, kvh, d, S)
    for t in range(S):
        assert abs(z[t, 0] - math.log(t + 1)) <= 1e-15 * (1 + math.log(t + 1))
