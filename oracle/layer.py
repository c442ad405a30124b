"""fp64 CPU oracle for one GPU's tensor-parallel share of a transformer layer's dense GEMM chain.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import or run this module. The product path never routes through it, and it shares no code with the
HIP library: it is the plain definition of what the sliced path must reproduce.

What is computed, and where it comes from:
  * The layer is a Megatron-style tensor-parallel MLP (and the attention input/output projections)
    seen from one rank: a column-parallel product, an activation, then a row-parallel product whose
    result is a partial sum that the tensor-parallel group would add up. (Domino page, Abstract: the
    system being sped up is Megatron-LM tensor-parallel LLM training; builds-on list: "Megatron-LM:
    Training Multi-Billion Parameter Language Models Using Model Parallelism".)
  * The activation is the GELU x*Phi(x) for the GPT family, and the SwiGLU gate silu(x W_g) * (x W_u)
    for the Llama family. (Domino page, builds-on list: "GLU Variants Improve Transformer".)
  * Slicing the batch into independent pieces and overlapping their hand-off with later compute
    changes no value: the pieces are independent (Domino page, Abstract), and overlap reorders
    operators without changing training semantics (DHelix review, "If this is right"). So the oracle
    computes only the unsliced definition; a sliced result is judged against the same numbers.

Storage convention (matches the inputs): weights are [out_features][in_features]; activations are
[tokens][features]; every array is float64, widened exactly from the bf16 inputs.

Nothing here rounds to bf16: every intermediate stays fp64.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np
from scipy.special import erf

_INV_SQRT2 = 1.0 / math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


# ----------------------------------------------------------------------------------- activations
def gelu(u: np.ndarray) -> np.ndarray:
    """GELU(u) = u * Phi(u), Phi the standard normal CDF = (1 + erf(u / sqrt 2)) / 2."""
    return 0.5 * u * (1.0 + erf(u * _INV_SQRT2))


def gelu_prime(u: np.ndarray) -> np.ndarray:
    """d/du [u Phi(u)] = Phi(u) + u phi(u), phi the standard normal density."""
    return 0.5 * (1.0 + erf(u * _INV_SQRT2)) + u * np.exp(-0.5 * u * u) * _INV_SQRT_2PI


def sigmoid(g: np.ndarray) -> np.ndarray:
    """1 / (1 + e^-g), evaluated without overflow for large |g|."""
    g = np.asarray(g, dtype=np.float64)
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-g[pos]))
    e = np.exp(g[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def silu(g: np.ndarray) -> np.ndarray:
    """Swish with beta = 1: g * sigmoid(g)."""
    return g * sigmoid(g)


def silu_prime(g: np.ndarray) -> np.ndarray:
    """d/dg [g s(g)] = s(g) (1 + g (1 - s(g)))."""
    s = sigmoid(g)
    return s * (1.0 + g * (1.0 - s))


# ----------------------------------------------------------------------------------------- MLP
def _split_gate_up(U: np.ndarray):
    f = U.shape[1] // 2
    return U[:, :f], U[:, f:]


def activate(U: np.ndarray, act: str) -> np.ndarray:
    """H from the pre-activation U ([tokens][N1]); SwiGLU takes U = [G | V] column halves."""
    if act == "gelu":
        return gelu(U)
    if act == "swiglu":
        G, V = _split_gate_up(U)
        return silu(G) * V
    raise ValueError(act)


def mlp_fwd(X, W1, b1, W2, act: str) -> Dict[str, np.ndarray]:
    """Column-parallel up-projection, activation, row-parallel down-projection (one rank's share).

    X [M][h], W1 [N1][h], b1 [N1] or None, W2 [h][F']  ->  U [M][N1], H [M][F'], Z [M][h].
    Z is this rank's partial sum; the row-parallel bias is not part of it (it is added once, after
    the group's sum).
    """
    U = X @ W1.T
    if b1 is not None:
        U = U + b1[None, :]
    H = activate(U, act)
    Z = H @ W2.T
    return {"U": U, "H": H, "Z": Z}


def mlp_bwd(X, W1, W2, U, dY, act: str, with_bias: bool = False) -> Dict[str, np.ndarray]:
    """Backward of `mlp_fwd` given the saved pre-activation U and the upstream gradient dY [M][h].

    Returns dX [M][h] (this rank's partial sum of the input gradient), dW1 [N1][h], dW2 [h][F'],
    db1 [N1] (when with_bias), plus the intermediates dU [M][N1] and H [M][F'].
    """
    H = activate(U, act)
    dH = dY @ W2
    if act == "gelu":
        dU = dH * gelu_prime(U)
    elif act == "swiglu":
        G, V = _split_gate_up(U)
        dU = np.concatenate([dH * V * silu_prime(G), dH * silu(G)], axis=1)
    else:
        raise ValueError(act)
    out = {
        "dX": dU @ W1,
        "dW1": dU.T @ X,
        "dW2": dY.T @ H,
        "dU": dU,
        "H": H,
    }
    if with_bias:
        out["db1"] = dU.sum(axis=0)
    return out


# ----------------------------------------------------------------------- attention projections
def attnproj_fwd(X, Wqkv, bqkv, C, Wo) -> Dict[str, np.ndarray]:
    """QKV = X Wqkv^T (+ bias): column-parallel; Z = C Wo^T: row-parallel partial sum.

    X [M][h], Wqkv [(q+2kv)d][h], C [M][q d] (attention context, an input here), Wo [h][q d].
    """
    QKV = X @ Wqkv.T
    if bqkv is not None:
        QKV = QKV + bqkv[None, :]
    return {"QKV": QKV, "Z": C @ Wo.T}


def attnproj_bwd(X, Wqkv, dQKV, C, Wo, dY, with_bias: bool = False) -> Dict[str, np.ndarray]:
    """Backward of `attnproj_fwd` given dQKV (from the attention core) and dY (into the O projection).

    dC = dY Wo;  dWo = dY^T C;  dX = dQKV Wqkv (partial sum);  dWqkv = dQKV^T X.
    """
    out = {
        "dC": dY @ Wo,
        "dWo": dY.T @ C,
        "dX": dQKV @ Wqkv,
        "dWqkv": dQKV.T @ X,
    }
    if with_bias:
        out["dbqkv"] = dQKV.sum(axis=0)
    return out


def as_f64(t) -> np.ndarray:
    """Exact widening of a bf16/fp32 torch tensor (CPU) or array to float64."""
    if hasattr(t, "detach"):
        return t.detach().to("cpu").float().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)
