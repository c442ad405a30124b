"""Seeded synthetic inputs for the sliced tensor-parallel layer shard.

This module only draws random tensors and names the workload shapes. It holds none of the layer's
arithmetic: both the HIP path and the fp64 checker receive exactly the bf16 tensors made here.

Workload shapes follow the model families the pages train: GPT-3 and Llama 2/3 (Domino page, builds-on
list: "Language Models are Few-Shot Learners", "Llama 2"; FiCCO page, builds-on list: "The Llama 3 Herd
of Models"), split Megatron-style over a simulated tensor-parallel group (Domino page, Abstract: the
comparison baseline is Megatron-LM).

Storage convention (all row-major, bf16):
  X, X_mlp, C, dY, dY_attn : [tokens][features]
  W1      : [N1][hidden]        N1 = F' (GeLU) or 2F' with rows [gate | up] (SwiGLU)
  b1      : [N1]                (GPT-style workloads only)
  W2      : [hidden][F']
  Wqkv    : [(q + 2 kv) d][hidden], rows ordered [Q heads | K heads | V heads]
  Wo      : [hidden][q d]
  U_saved : [tokens][N1]        pre-activation handed to the backward pass
Weights use the [out_features][in_features] layout of a linear layer, so the forward products read
both operands along the reduction dimension.

A value drawn as N(0, s) has standard deviation s. Each tensor is drawn in fp32 from its own
torch.Generator seeded with 1000 * workload_index + tensor_id, scaled, then rounded to bf16 (RNE).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Tuple

import torch

# tensor ids used in the seed formula
TENSOR_IDS = {
    "X": 1, "W1": 2, "b1": 3, "W2": 4, "b2": 5, "Wqkv": 6, "C": 7, "Wo": 8,
    "dY": 9, "dQKV": 10, "X_mlp": 11, "dY_attn": 12, "U_saved": 13,
}


@dataclass(frozen=True)
class Workload:
    key: str
    index: int                 # seed base: 1000 * index + tensor id
    tokens: int                # M
    hidden: int                # h
    ffn: int                   # full FFN width F; the shard holds F' = ffn // tp
    tp: int                    # simulated tensor-parallel group size
    act: str                   # "gelu" | "swiglu"
    bias: bool                 # b1 present (GPT family)
    row_slices: int            # r
    col_slices: int            # c
    heads: int = 0             # full-model query heads (0: no attention projections)
    kv_heads: int = 0
    head_dim: int = 0
    backward: bool = False
    note: str = ""

    @property
    def ffn_shard(self) -> int:
        return self.ffn // self.tp

    @property
    def n1(self) -> int:
        return 2 * self.ffn_shard if self.act == "swiglu" else self.ffn_shard

    @property
    def q_heads_shard(self) -> int:
        return self.heads // self.tp

    @property
    def kv_heads_shard(self) -> int:
        return max(1, self.kv_heads // self.tp) if self.kv_heads else 0

    @property
    def qkv_width(self) -> int:
        return (self.q_heads_shard + 2 * self.kv_heads_shard) * self.head_dim

    @property
    def ctx_width(self) -> int:
        return self.q_heads_shard * self.head_dim

    @property
    def has_attn(self) -> bool:
        return self.heads > 0

    def gemm_flops(self) -> Dict[str, int]:
        """2*M*N*K for every product the workload runs (forward, and backward if enabled)."""
        M, h, Fp, N1 = self.tokens, self.hidden, self.ffn_shard, self.n1
        f = {"mlp_up": 2 * M * N1 * h, "mlp_down": 2 * M * h * Fp}
        if self.has_attn:
            f["qkv"] = 2 * M * self.qkv_width * h
            f["o"] = 2 * M * h * self.ctx_width
        if self.backward:
            for k in list(f):
                f[k + "_dgrad"] = f[k]
                f[k + "_wgrad"] = f[k]
        return f


WORKLOADS: Dict[str, Workload] = {
    "tiny_gpt_mlp": Workload(
        "tiny_gpt_mlp", 1, tokens=256, hidden=512, ffn=2048, tp=4, act="gelu", bias=True,
        row_slices=2, col_slices=2, note="tiny GPT-style MLP shard, forward"),
    "gpt3_2.7b_mlp": Workload(
        "gpt3_2.7b_mlp", 2, tokens=8192, hidden=2560, ffn=10240, tp=2, act="gelu", bias=True,
        row_slices=2, col_slices=1, note="GPT-3 2.7B MLP shard at TP 1/2, forward"),
    "llama2_7b_mlp": Workload(
        "llama2_7b_mlp", 3, tokens=8192, hidden=4096, ffn=11008, tp=4, act="swiglu", bias=False,
        row_slices=4, col_slices=2, note="Llama-2 7B SwiGLU MLP shard at TP 1/4, forward"),
    "llama2_13b_layer": Workload(
        "llama2_13b_layer", 4, tokens=8192, hidden=5120, ffn=13824, tp=8, act="swiglu", bias=False,
        row_slices=4, col_slices=1, heads=40, kv_heads=40, head_dim=128, backward=True,
        note="Llama-2 13B layer shard at TP 1/8, forward and backward"),
    "llama3_70b_layer": Workload(
        "llama3_70b_layer", 5, tokens=16384, hidden=8192, ffn=28672, tp=8, act="swiglu", bias=False,
        row_slices=8, col_slices=2, heads=64, kv_heads=8, head_dim=128, backward=True,
        note="Llama-3 70B layer shard at TP 1/8, forward and backward"),
}


def custom(key: str, index: int, **kw) -> Workload:
    """A test workload with explicit sizes (for ragged and edge-case shapes)."""
    base = dict(tokens=64, hidden=64, ffn=64, tp=1, act="gelu", bias=False, row_slices=1,
                col_slices=1)
    base.update(kw)
    return Workload(key, index, **base)


def randn_bf16(shape: Tuple[int, ...], std: float, seed: int) -> torch.Tensor:
    """N(0, std) drawn in fp32 from a generator seeded with `seed`, rounded to bf16 (RNE)."""
    g = torch.Generator().manual_seed(int(seed))
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def make_inputs(w: Workload, which: Optional[Tuple[str, ...]] = None) -> Dict[str, torch.Tensor]:
    """CPU bf16 tensors for workload `w`. `which` restricts the set (default: all the workload uses)."""
    M, h, N1, Fp = w.tokens, w.hidden, w.n1, w.ffn_shard
    spec = {
        "X_mlp": ((M, h), 1.0),
        "W1": ((N1, h), 0.02),
        "W2": ((h, Fp), 0.02),
    }
    if w.bias:
        spec["b1"] = ((N1,), 0.01)
        spec["b2"] = ((h,), 0.01)
    if w.has_attn:
        spec["X"] = ((M, h), 1.0)
        spec["Wqkv"] = ((w.qkv_width, h), 0.02)
        spec["C"] = ((M, w.ctx_width), 1.0)
        spec["Wo"] = ((h, w.ctx_width), 0.02)
    if w.backward:
        spec["dY"] = ((M, h), 0.01)
        spec["U_saved"] = ((M, N1), 0.02 * math.sqrt(h))
        if w.has_attn:
            spec["dY_attn"] = ((M, h), 0.01)
            spec["dQKV"] = ((M, w.qkv_width), 0.01)
    names = which if which is not None else tuple(spec)
    out = {}
    for name in names:
        shape, std = spec[name]
        out[name] = randn_bf16(shape, std, 1000 * w.index + TENSOR_IDS[name])
    return out
