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
