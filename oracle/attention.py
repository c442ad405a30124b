"""fp64 CPU oracle of the attention core between the QKV and the output projections.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import or run this module. The product path never routes through it, and it shares no code with the
HIP library.

What is computed: causal (decoder) softmax attention of one tensor-parallel rank's heads, the
operation the FlashAttention papers in the Domino page's builds-on list compute exactly (they
reorganise the same softmax attention into tiles without changing its value). For a batch of
sequences stored as contiguous runs of `seq_len` token rows (batch-major rows, as the layer's
tokens are), query head h of this rank reads key/value head g = h // (q_heads / kv_heads) (grouped
KV heads; one KV head serves all query heads when kv_heads = 1), and for token t of a sequence

    C[t, h] = sum over s <= t of softmax_s(Q[t, h] . K[s, g] / sqrt(head_dim)) V[s, g]

with s, t positions within the same sequence. QKV rows hold [Q heads | K heads | V heads], each head
`head_dim` contiguous columns (the projection's column layout); C rows hold the query heads in order.
Everything stays fp64.

The backward pass is the gradient of the same function (chain rule through the softmax; the
FlashAttention papers compute the same gradient in tiles): for L with dL/dC = dC, per sequence,
query head h and its key/value head g, with P[t, s] the softmax weights above (0 for s > t),

    dV[s, g] += sum_t P[t, s] dC[t, h]                        (over the group's query heads h)
    dP[t, s]  = dC[t, h] . V[s, g]
    dA[t, s]  = P[t, s] (dP[t, s] - sum_r P[t, r] dP[t, r])   (A = the scaled scores)
    dQ[t, h]  = sum_s dA[t, s] K[s, g] / sqrt(head_dim)
    dK[s, g] += sum_t dA[t, s] Q[t, h] / sqrt(head_dim)
"""
from __future__ import annotations

import math

import numpy as np


def split_qkv(QKV: np.ndarray, q_heads: int, kv_heads: int, head_dim: int):
    """Q [M][q][d], K [M][kv][d], V [M][kv][d] views of a [M][(q + 2 kv) d] array."""
    M = QKV.shape[0]
    q = QKV[:, : q_heads * head_dim].reshape(M, q_heads, head_dim)
    k = QKV[:, q_heads * head_dim: (q_heads + kv_heads) * head_dim].reshape(M, kv_heads, head_dim)
    v = QKV[:, (q_heads + kv_heads) * head_dim: (q_heads + 2 * kv_heads) * head_dim].reshape(M, kv_heads, head_dim)
    return q, k, v


def attn_core_fwd(QKV: np.ndarray, q_heads: int, kv_heads: int, head_dim: int, seq_len: int) -> np.ndarray:
    """C [M][q_heads * head_dim] from QKV [M][(q_heads + 2 kv_heads) head_dim]; M a multiple of seq_len."""
    M = QKV.shape[0]
    assert M % seq_len == 0 and q_heads % kv_heads == 0
    q, k, v = split_qkv(np.asarray(QKV, dtype=np.float64), q_heads, kv_heads, head_dim)
    group = q_heads // kv_heads
    scale = 1.0 / math.sqrt(head_dim)
    C = np.empty((M, q_heads, head_dim), dtype=np.float64)
    causal = np.tril(np.ones((seq_len, seq_len), dtype=bool))
    for b in range(M // seq_len):
        rows = slice(b * seq_len, (b + 1) * seq_len)
        for h in range(q_heads):
            g = h // group
            s = (q[rows, h, :] @ k[rows, g, :].T) * scale          # [t][s]
            s = np.where(causal, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            C[rows, h, :] = p @ v[rows, g, :]
    return C.reshape(M, q_heads * head_dim)


def attn_core_bwd(QKV: np.ndarray, dC: np.ndarray, q_heads: int, kv_heads: int, head_dim: int,
                  seq_len: int) -> np.ndarray:
    """dQKV [M][(q_heads + 2 kv_heads) head_dim] (the [dQ | dK | dV] layout of QKV) from the forward's
    input QKV and the gradient dC [M][q_heads head_dim] of its output."""
    M = QKV.shape[0]
    assert M % seq_len == 0 and q_heads % kv_heads == 0
    q, k, v = split_qkv(np.asarray(QKV, dtype=np.float64), q_heads, kv_heads, head_dim)
    dc = np.asarray(dC, dtype=np.float64).reshape(M, q_heads, head_dim)
    group = q_heads // kv_heads
    scale = 1.0 / math.sqrt(head_dim)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    causal = np.tril(np.ones((seq_len, seq_len), dtype=bool))
    for b in range(M // seq_len):
        rows = slice(b * seq_len, (b + 1) * seq_len)
        for h in range(q_heads):
            g = h // group
            a = (q[rows, h, :] @ k[rows, g, :].T) * scale
            a = np.where(causal, a, -np.inf)
            a = a - a.max(axis=1, keepdims=True)
            p = np.exp(a)
            p /= p.sum(axis=1, keepdims=True)                   # [t][s]
            dv[rows, g, :] += p.T @ dc[rows, h, :]
            dp = dc[rows, h, :] @ v[rows, g, :].T                # [t][s]
            da = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[rows, h, :] = (da @ k[rows, g, :]) * scale
            dk[rows, g, :] += (da.T @ q[rows, h, :]) * scale
    return np.concatenate([dq.reshape(M, -1), dk.reshape(M, -1), dv.reshape(M, -1)], axis=1)


def attn_core_lse(QKV: np.ndarray, q_heads: int, kv_heads: int, head_dim: int, seq_len: int) -> np.ndarray:
    """Natural log of each row's softmax denominator, log sum over s <= t of exp(Q[t, h] . K[s, g] /
    sqrt(head_dim)): [M][q_heads] (the normaliser a tiled forward pass keeps for its backward)."""
    M = QKV.shape[0]
    q, k, _ = split_qkv(np.asarray(QKV, dtype=np.float64), q_heads, kv_heads, head_dim)
    group = q_heads // kv_heads
    scale = 1.0 / math.sqrt(head_dim)
    out = np.empty((M, q_heads), dtype=np.float64)
    causal = np.tril(np.ones((seq_len, seq_len), dtype=bool))
    for b in range(M // seq_len):
        rows = slice(b * seq_len, (b + 1) * seq_len)
        for h in range(q_heads):
            a = (q[rows, h, :] @ k[rows, h // group, :].T) * scale
            a = np.where(causal, a, -np.inf)
            mx = a.max(axis=1, keepdims=True)
            out[rows, h] = (mx + np.log(np.exp(a - mx).sum(axis=1, keepdims=True)))[:, 0]
    return out
