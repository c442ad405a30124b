"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle, plus the exact identities
that slicing and overlap must keep (Domino page, Abstract: the pieces are independent; DHelix review,
"If this is right": overlap leaves semantics unchanged)."""
import numpy as np
import pytest
import torch

from comm_overlap_amd import synth
from oracle import layer as L
import gpu_cases as G

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from comm_overlap_amd import tpslice as T

f64 = L.as_f64

# Small shapes that span several 256-wide tiles with ragged tails in every dimension.
SMALL_GELU = synth.custom("small_gelu", 901, tokens=640, hidden=528, ffn=328, tp=1, act="gelu", bias=True,
                          row_slices=2, col_slices=2, backward=True)
SMALL_SWIGLU = synth.custom("small_swiglu", 902, tokens=576, hidden=272, ffn=400, tp=2, act="swiglu",
                            bias=False, row_slices=3, col_slices=2, backward=True)
SMALL_ATTN = synth.custom("small_attn", 903, tokens=520, hidden=264, ffn=64, tp=2, act="gelu", bias=False,
                          row_slices=2, col_slices=1, heads=6, kv_heads=2, head_dim=40, backward=True)


def _print_case(name, **kw):
    print(f"[case] {name} {kw}", flush=True)


@pytest.mark.parametrize("tile", ["256x256", "128x128", "256x320", "128x320", "128x256", "128x128w8", "256x224w4"])
@pytest.mark.parametrize("w", [SMALL_GELU, SMALL_SWIGLU], ids=lambda w: w.key)
def test_mlp_fwd_small(w, tile):
    _print_case("mlp_fwd", key=w.key, tile=tile)
    inp = synth.make_inputs(w)
    plan = T.plan_for(w, tile=tile)
    out = G.run_mlp_fwd(plan, inp)
    ref = G.oracle_mlp_fwd(inp, w.act)
    G.assert_parity(out["Z"], ref["Z"], "Z")
    G.assert_parity(out["U"], ref["U"], "U")
    assert torch.equal(out["Zh"], out["Z"])


# Forward products for the four-wave tiles (k a multiple of 64): whole tiles with an even number of
# k blocks, and ragged rows and columns with an odd number (the loop then runs one all-zero block).
WHOLE_GELU = synth.custom("whole_gelu", 904, tokens=1024, hidden=1280, ffn=2560, tp=1, act="gelu", bias=True,
                          row_slices=2, col_slices=1)
WHOLE_SWIGLU = synth.custom("whole_swiglu", 905, tokens=1024, hidden=1280, ffn=5120, tp=2, act="swiglu",
                            bias=False, row_slices=2, col_slices=1)
RAGGED64_GELU = synth.custom("ragged64_gelu", 906, tokens=1000, hidden=1216, ffn=1344, tp=1, act="gelu",
                             bias=True, row_slices=2, col_slices=2)
RAGGED64_SWIGLU = synth.custom("ragged64_swiglu", 907, tokens=744, hidden=704, ffn=2752, tp=2, act="swiglu",
                               bias=True, row_slices=3, col_slices=1)


@pytest.mark.parametrize("w", [WHOLE_GELU, WHOLE_SWIGLU, RAGGED64_GELU, RAGGED64_SWIGLU], ids=lambda w: w.key)
def test_four_wave_tiles(w):
    """The software-pipelined four-wave tiles against the oracle, and bit for bit against the
    eight-wave 256 x 256 tile (same k order), twice in a row."""
    inp = synth.make_inputs(w)
    ref = G.oracle_mlp_fwd(inp, w.act)
    base = G.run_mlp_fwd(T.plan_for(w, tile="256x256"), inp)
    for tile in ("256x256w4", "256x160w4", "256x320w4", "256x224w4", "auto", "256x256w4", "256x224w4"):
        _print_case("four_wave", key=w.key, tile=tile)
        out = G.run_mlp_fwd(T.plan_for(w, tile=tile), inp)
        G.assert_parity(out["Z"], ref["Z"], "Z")
        G.assert_parity(out["U"], ref["U"], "U")
        assert torch.equal(out["Z"], base["Z"]), tile
        assert torch.equal(out["U"], base["U"]), tile
        assert torch.equal(out["Zh"], out["Z"]), tile


# Backward products for the four-wave tiles: every k (h, the FFN shard, the token count) a multiple
# of 64, with odd k block counts and ragged rows and columns; operands stored across k (weights in
# the activation gradients, both operands of the weight gradients) go through transposing reads.
# 256 x 160 takes the activation gradients with a bf16 or GeLU-gradient epilogue, its B tile padded
# to 256 columns in LDS (dX: 1216, 1280, 1344 columns; GeLU dH: 1344).
BWD64_GELU = synth.custom("bwd64_gelu", 910, tokens=1088, hidden=1216, ffn=1344, tp=1, act="gelu", bias=True,
                          row_slices=2, col_slices=2, backward=True)
BWD64_SWIGLU = synth.custom("bwd64_swiglu", 911, tokens=1024, hidden=1280, ffn=2752, tp=2, act="swiglu",
                            bias=False, row_slices=2, col_slices=1, backward=True)
BWD64_ATTN = synth.custom("bwd64_attn", 912, tokens=1088, hidden=1344, ffn=64, tp=2, act="gelu", bias=False,
                          row_slices=2, col_slices=1, heads=6, kv_heads=2, head_dim=64, backward=True)


@pytest.mark.parametrize("w", [BWD64_GELU, BWD64_SWIGLU], ids=lambda w: w.key)
def test_four_wave_tiles_mlp_backward(w):
    """MLP backward with the four-wave tiles (activation gradients, weight gradients and split
    partial products) against the oracle, and bit for bit against the eight-wave 256 x 256 tile,
    twice in a row."""
    inp = synth.make_inputs(w)
    ref = L.mlp_bwd(f64(inp["X_mlp"]), f64(inp["W1"]), f64(inp["W2"]), f64(inp["U_saved"]), f64(inp["dY"]),
                    w.act, with_bias=w.bias)
    base = G.run_mlp_bwd(T.plan_for(w, tile="256x256"), inp, with_bias=w.bias)
    keys = ("dX", "dW1", "dW2") + (("db1",) if w.bias else ())
    for tile in ("256x256w4", "256x160w4", "auto", "256x256w4", "256x160w4"):
        _print_case("four_wave_bwd", key=w.key, tile=tile)
        out = G.run_mlp_bwd(T.plan_for(w, tile=tile), inp, with_bias=w.bias)
        for k in keys:
            G.assert_parity(out[k], ref[k], k)
            assert torch.equal(out[k], base[k]), (tile, k)
        assert torch.equal(out["dXh"], out["dX"]), tile


def test_four_wave_tiles_attn_backward():
    w = BWD64_ATTN
    inp = synth.make_inputs(w)
    ref = L.attnproj_bwd(f64(inp["X"]), f64(inp["Wqkv"]), f64(inp["dQKV"]), f64(inp["C"]), f64(inp["Wo"]),
                         f64(inp["dY_attn"]), with_bias=True)
    base = G.run_attn_bwd(T.plan_for(w, tile="256x256"), inp, with_bias=True)
    for tile in ("256x256w4", "256x160w4", "auto"):
        _print_case("four_wave_attn_bwd", key=w.key, tile=tile)
        out = G.run_attn_bwd(T.plan_for(w, tile=tile), inp, with_bias=True)
        for k in ("dX", "dC", "dWqkv", "dWo", "dbqkv"):
            G.assert_parity(out[k], ref[k], k)
            assert torch.equal(out[k], base[k]), (tile, k)


AUTO = synth.custom("auto_slices", 909, tokens=2048, hidden=1024, ffn=4096, tp=1, act="gelu", bias=True,
                    row_slices=1, col_slices=1)


@pytest.mark.parametrize("gbps", [0.0, 25.0])
def test_automatic_slice_counts(gbps):
    """A plan that chooses its own slice counts computes the same layer (the slower assumed
    hand-off makes it slice this workload)."""
    w = AUTO
    inp = synth.make_inputs(w)
    plan = T.plan_for(w, n_row_slices=0, n_col_slices=0, handoff_gbps=gbps)
    _print_case("auto_slices", key=w.key, gbps=gbps, r=plan.info.n_row_slices, c=plan.info.n_col_slices)
    if gbps == 25.0:
        assert plan.info.n_row_slices * plan.info.n_col_slices > 1
    out = G.run_mlp_fwd(plan, inp)
    ref = G.oracle_mlp_fwd(inp, w.act)
    G.assert_parity(out["Z"], ref["Z"], "Z")
    assert torch.equal(out["Zh"], out["Z"])


@pytest.mark.parametrize("mode", ["dma", "kernel", "pipelined"])
def test_two_strands_match_separate_calls(mode):
    """The forward of one micro-batch beside the backward of another, each a serialized plan on a
    stream of its own (the two strands of the micro-batch co-execution page, "What carries the
    argument"; as bench.py --strands 2 runs them), gives the bits of the same calls run one after
    the other."""
    w = SMALL_ATTN
    _print_case("two_strands", key=w.key, mode=mode)
    inp = synth.make_inputs(w)
    if mode == "pipelined":  # worker 0 is the strand's stream; DMA copies on a copy stream each
        kw = dict(pipeline=True, caller_worker=True, n_streams=1, n_copy_streams=1)
    else:
        kw = dict(serialize=True, copy_blit=mode == "kernel")
    # each strand's plan has copy streams of its own, so that the two strands' copies overlap
    fwd_plan = T.plan_for(w, streams=T.Streams.new(0, 1), **kw)
    bwd_plan = T.plan_for(w, streams=T.Streams.new(0, 1), **kw)

    def forward(sync):
        return G.run_attn_fwd(fwd_plan, inp, sync=sync), G.run_mlp_fwd(fwd_plan, inp, sync=sync)

    def backward(sync):
        return (G.run_mlp_bwd(bwd_plan, inp, with_bias=w.bias, sync=sync),
                G.run_attn_bwd(bwd_plan, inp, with_bias=False, sync=sync))

    ref = forward(True) + backward(True)
    fwd_plan.handoff_wait()
    bwd_plan.handoff_wait()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(sa):
        got_f = forward(False)
        fwd_plan.handoff_wait(sa)
    with torch.cuda.stream(sb):
        got_b = backward(False)
        bwd_plan.handoff_wait(sb)
    torch.cuda.synchronize()
    for r, g in zip(ref, got_f + got_b):
        for k, v in r.items():
            if v is not None:
                assert torch.equal(v, g[k]), k


def test_mlp_fwd_tiny_workload():
    w = synth.WORKLOADS["tiny_gpt_mlp"]
    _print_case("mlp_fwd", key=w.key)
    inp = synth.make_inputs(w)
    plan = T.plan_for(w)
    out = G.run_mlp_fwd(plan, inp)
    ref = G.oracle_mlp_fwd(inp, w.act)
    G.assert_parity(out["Z"], ref["Z"], "Z")
    G.assert_parity(out["U"], ref["U"], "U")
    assert torch.equal(out["Zh"], out["Z"])


@pytest.mark.parametrize("w", [SMALL_GELU, SMALL_SWIGLU, synth.WORKLOADS["tiny_gpt_mlp"]], ids=lambda w: w.key)
def test_slicing_is_bit_exact(w):
    """Sliced == unsliced, serialized == concurrent, blit copy == DMA copy, repeat == first run."""
    _print_case("bitexact", key=w.key)
    inp = synth.make_inputs(w)
    base = G.run_mlp_fwd(T.plan_for(w, n_row_slices=1, n_col_slices=1), inp)
    for kw in [dict(), dict(serialize=True), dict(copy_blit=True), dict(n_streams=3, n_copy_streams=2),
               dict(tile="256x256"), dict(tile="128x128"), dict(tile="256x320"), dict(tile="128x320"),
               dict(tile="128x256"), dict(tile="128x128w8")]:
        out = G.run_mlp_fwd(T.plan_for(w, **kw), inp)
        assert torch.equal(out["Z"], base["Z"]), kw
        assert torch.equal(out["U"], base["U"]), kw
        assert torch.equal(out["Zh"], base["Z"]), kw
    again = G.run_mlp_fwd(T.plan_for(w), inp)
    assert torch.equal(again["Z"], base["Z"])


def test_closed_forms_exact():
    w = SMALL_GELU
    inp = synth.make_inputs(w)
    plan = T.plan_for(w)
    # W2 = 0  =>  Z = 0 exactly
    z = dict(inp, W2=torch.zeros_like(inp["W2"]))
    out = G.run_mlp_fwd(plan, z)
    assert torch.count_nonzero(out["Z"].float()) == 0
    # W1 = 0  =>  every row of Z is the same (act(b1) W2^T), bit for bit
    z = dict(inp, W1=torch.zeros_like(inp["W1"]))
    out = G.run_mlp_fwd(plan, z)
    assert torch.equal(out["Z"], out["Z"][:1].expand_as(out["Z"]))
    ref = G.oracle_mlp_fwd({k: v[:1] if k == "X_mlp" else v for k, v in z.items()}, w.act)
    G.assert_parity(out["Z"][:1], ref["Z"], "Z row")
    # W2 scaled by 2^3  =>  Z scaled by 2^3 bitwise (exact in binary floating point)
    base = G.run_mlp_fwd(plan, inp)
    out = G.run_mlp_fwd(plan, dict(inp, W2=inp["W2"] * 8))
    assert torch.equal(out["Z"], base["Z"] * 8)


def test_row_permutation_commutes():
    """Permuting token rows permutes output rows, bitwise (rows are independent)."""
    w = SMALL_SWIGLU
    inp = synth.make_inputs(w)
    plan = T.plan_for(w)
    perm = torch.randperm(w.tokens, generator=torch.Generator().manual_seed(5))
    base = G.run_mlp_fwd(plan, inp)
    out = G.run_mlp_fwd(plan, dict(inp, X_mlp=inp["X_mlp"][perm].contiguous()))
    assert torch.equal(out["Z"], base["Z"][perm.cuda()])


@pytest.mark.parametrize("bias", [True, False])
def test_attnproj_fwd_small(bias):
    w = SMALL_ATTN
    _print_case("attn_fwd", key=w.key, bias=bias)
    inp = synth.make_inputs(w)
    bqkv = synth.randn_bf16((w.qkv_width,), 0.01, 77) if bias else None
    plan = T.plan_for(w)
    out = G.run_attn_fwd(plan, inp, bias=bqkv)
    ref = L.attnproj_fwd(f64(inp["X"]), f64(inp["Wqkv"]), f64(bqkv) if bias else None, f64(inp["C"]),
                         f64(inp["Wo"]))
    G.assert_parity(out["QKV"], ref["QKV"], "QKV")
    G.assert_parity(out["Z"], ref["Z"], "Z")
    assert torch.equal(out["Zh"], out["Z"])
    for kw in (dict(n_row_slices=1), dict(tile="256x256"), dict(tile="128x128"), dict(tile="256x320"),
               dict(tile="128x320"), dict(tile="128x256")):
        one = G.run_attn_fwd(T.plan_for(w, **kw), inp, bias=bqkv)
        assert torch.equal(one["Z"], out["Z"]) and torch.equal(one["QKV"], out["QKV"]), kw


@pytest.mark.parametrize("w", [SMALL_GELU, SMALL_SWIGLU], ids=lambda w: w.key)
def test_mlp_bwd_small(w):
    _print_case("mlp_bwd", key=w.key)
    inp = synth.make_inputs(w)
    plan = T.plan_for(w)
    out = G.run_mlp_bwd(plan, inp, with_bias=w.bias)
    ref = L.mlp_bwd(f64(inp["X_mlp"]), f64(inp["W1"]), f64(inp["W2"]), f64(inp["U_saved"]), f64(inp["dY"]),
                    w.act, with_bias=w.bias)
    G.assert_parity(out["dX"], ref["dX"], "dX")
    G.assert_parity(out["dW1"], ref["dW1"], "dW1")
    G.assert_parity(out["dW2"], ref["dW2"], "dW2")
    if w.bias:
        G.assert_parity(out["db1"], ref["db1"], "db1")
    assert torch.equal(out["dXh"], out["dX"])
    # either block tile gives the same bits (same k order)
    for tile in ("256x256", "128x128", "128x256", "128x128w8"):
        o2 = G.run_mlp_bwd(T.plan_for(w, tile=tile), inp, with_bias=w.bias)
        for k in ("dX", "dW1", "dW2", "db1"):
            if out[k] is not None:
                assert torch.equal(o2[k], out[k]), (tile, k)
    # accumulate = 1 adds to what is there; the token sum is not split, so it matches bitwise a
    # run whose fp32 accumulators start from the same values
    init = tuple(torch.randn_like(t) if t is not None else None for t in (out["dW1"], out["dW2"], out["db1"]))
    acc = G.run_mlp_bwd(plan, inp, with_bias=w.bias, accumulate=True, init=init)
    G.assert_parity(acc["dW1"], f64(init[0].cpu()) + ref["dW1"], "dW1 accumulated")
    G.assert_parity(acc["dW2"], f64(init[1].cpu()) + ref["dW2"], "dW2 accumulated")
    # sliced == unsliced, serialized == concurrent
    for kw in [dict(n_row_slices=1, n_col_slices=1), dict(serialize=True)]:
        o2 = G.run_mlp_bwd(T.plan_for(w, **kw), inp, with_bias=w.bias)
        for k in ("dX", "dW1", "dW2", "db1"):
            if out[k] is not None:
                assert torch.equal(o2[k], out[k]), (kw, k)


@pytest.mark.parametrize("bias", [True, False])
def test_attnproj_bwd_small(bias):
    w = SMALL_ATTN
    _print_case("attn_bwd", key=w.key, bias=bias)
    inp = synth.make_inputs(w)
    plan = T.plan_for(w)
    out = G.run_attn_bwd(plan, inp, with_bias=bias)
    ref = L.attnproj_bwd(f64(inp["X"]), f64(inp["Wqkv"]), f64(inp["dQKV"]), f64(inp["C"]), f64(inp["Wo"]),
                         f64(inp["dY_attn"]), with_bias=bias)
    for k in ("dX", "dC", "dWqkv", "dWo") + (("dbqkv",) if bias else ()):
        G.assert_parity(out[k], ref[k], k)
    assert torch.equal(out["dXh"], out["dX"])
    for kw in (dict(tile="256x256"), dict(tile="128x128"), dict(tile="128x256"), dict(tile="128x128w8"),
               dict(n_row_slices=1)):
        o2 = G.run_attn_bwd(T.plan_for(w, **kw), inp, with_bias=bias)
        for k in ("dX", "dC", "dWqkv", "dWo") + (("dbqkv",) if bias else ()):
            assert torch.equal(o2[k], out[k]), (kw, k)


# Long token sums with narrow outputs: the weight gradients (and dC) are split along k, their fp32
# partial products reduced in split order.
SPLIT_K = synth.custom("split_k", 906, tokens=2048, hidden=264, ffn=200, tp=1, act="gelu", bias=True,
                       row_slices=2, col_slices=1, heads=6, kv_heads=2, head_dim=40, backward=True)


def test_split_k_backward():
    w = SPLIT_K
    _print_case("split_k", key=w.key)
    inp = synth.make_inputs(w)
    plan = T.plan_for(w)
    out = G.run_mlp_bwd(plan, inp, with_bias=True)
    ref = L.mlp_bwd(f64(inp["X_mlp"]), f64(inp["W1"]), f64(inp["W2"]), f64(inp["U_saved"]), f64(inp["dY"]),
                    w.act, with_bias=True)
    for k in ("dX", "dW1", "dW2", "db1"):
        G.assert_parity(out[k], ref[k], k)
    init = (torch.randn_like(out["dW1"]), torch.randn_like(out["dW2"]), torch.randn_like(out["db1"]))
    acc = G.run_mlp_bwd(plan, inp, with_bias=True, accumulate=True, init=init)
    G.assert_parity(acc["dW1"], f64(init[0].cpu()) + ref["dW1"], "dW1 accumulated")
    G.assert_parity(acc["dW2"], f64(init[1].cpu()) + ref["dW2"], "dW2 accumulated")
    aout = G.run_attn_bwd(plan, inp, with_bias=True)
    aref = L.attnproj_bwd(f64(inp["X"]), f64(inp["Wqkv"]), f64(inp["dQKV"]), f64(inp["C"]), f64(inp["Wo"]),
                          f64(inp["dY_attn"]), with_bias=True)
    for k in ("dX", "dC", "dWqkv", "dWo", "dbqkv"):
        G.assert_parity(aout[k], aref[k], k)
    # the split depends on the product's shape only: slicing, tiles and streams keep the bits
    for kw in (dict(n_row_slices=1), dict(tile="128x128"), dict(tile="256x256"), dict(serialize=True)):
        o2 = G.run_mlp_bwd(T.plan_for(w, **kw), inp, with_bias=True)
        for k in ("dX", "dW1", "dW2", "db1"):
            assert torch.equal(o2[k], out[k]), (kw, k)
        a2 = G.run_attn_bwd(T.plan_for(w, **kw), inp, with_bias=True)
        for k in ("dX", "dC", "dWqkv", "dWo", "dbqkv"):
            assert torch.equal(a2[k], aout[k]), (kw, k)


# Weight gradients whose 256 x 256 tiles make one whole round of the 256 CUs plus a short tail
# (dW1: 17 tile rows of 16 tiles): only the tail rows are split along k, into one full round; the
# other rows run unsplit. Each element keeps one summation order, whatever the slicing or tile.
TAIL_SPLIT = [synth.custom("tail_split_swiglu", 913, tokens=2048, hidden=4096, ffn=2176, tp=1, act="swiglu",
                           bias=True, row_slices=2, col_slices=1, backward=True),
              synth.custom("tail_split_gelu", 914, tokens=2048, hidden=4096, ffn=4352, tp=1, act="gelu",
                           bias=True, row_slices=2, col_slices=2, backward=True)]


@pytest.mark.parametrize("w", TAIL_SPLIT, ids=lambda w: w.key)
def test_tail_split_weight_gradients(w):
    _print_case("tail_split", key=w.key)
    inp = synth.make_inputs(w)
    plan = T.plan_for(w)
    info = plan.info
    tail = info.split_rows()["dw1"]
    assert info.splits()["dw1"] > 1 and 0 < tail < info.n1 and (info.n1 - tail) % 256 == 0, info.split_rows()
    out = G.run_mlp_bwd(plan, inp, with_bias=True)
    ref = L.mlp_bwd(f64(inp["X_mlp"]), f64(inp["W1"]), f64(inp["W2"]), f64(inp["U_saved"]), f64(inp["dY"]),
                    w.act, with_bias=True)
    for k in ("dX", "dW1", "dW2", "db1"):
        G.assert_parity(out[k], ref[k], k)
    # both parts of dW1 on their own (the unsplit rows, the split tail)
    head = info.n1 - tail
    G.assert_parity(out["dW1"][:head], ref["dW1"][:head], "dW1 unsplit rows")
    G.assert_parity(out["dW1"][head:], ref["dW1"][head:], "dW1 tail rows")
    init = (torch.randn_like(out["dW1"]), torch.randn_like(out["dW2"]), torch.randn_like(out["db1"]))
    acc = G.run_mlp_bwd(plan, inp, with_bias=True, accumulate=True, init=init)
    G.assert_parity(acc["dW1"], f64(init[0].cpu()) + ref["dW1"], "dW1 accumulated")
    G.assert_parity(acc["dW2"], f64(init[1].cpu()) + ref["dW2"], "dW2 accumulated")
    for kw in (dict(n_row_slices=1), dict(tile="128x128"), dict(tile="256x256"), dict(serialize=True)):
        o2 = G.run_mlp_bwd(T.plan_for(w, **kw), inp, with_bias=True)
        for k in ("dX", "dW1", "dW2", "db1"):
            assert torch.equal(o2[k], out[k]), (kw, k)


# A long reduction (h = 2048) with narrow projections: the up-projection of each row slice, the QKV
# projection over all tokens and dH over each group of row slices are split along k; the split
# counts do not depend on the slicing.
SLICE_SPLIT = [synth.custom("slice_split_gelu", 907, tokens=1024, hidden=2048, ffn=264, tp=1, act="gelu",
                            bias=True, row_slices=2, col_slices=1, heads=6, kv_heads=2, head_dim=40,
                            backward=True),
               synth.custom("slice_split_swiglu", 908, tokens=1024, hidden=2048, ffn=528, tp=2, act="swiglu",
                            bias=False, row_slices=4, col_slices=2, backward=True)]


@pytest.mark.parametrize("w", SLICE_SPLIT, ids=lambda w: w.key)
def test_split_k_slice_products(w):
    _print_case("slice_split", key=w.key)
    inp = synth.make_inputs(w)
    plan = T.plan_for(w)
    sp = plan.info.splits()
    assert sp["up"] > 1 and sp["dh"] > 1, sp
    out = G.run_mlp_fwd(plan, inp)
    ref = G.oracle_mlp_fwd(inp, w.act)
    G.assert_parity(out["Z"], ref["Z"], "Z")
    G.assert_parity(out["U"], ref["U"], "U")
    bo = G.run_mlp_bwd(plan, inp, with_bias=w.bias)
    rb = L.mlp_bwd(f64(inp["X_mlp"]), f64(inp["W1"]), f64(inp["W2"]), f64(inp["U_saved"]), f64(inp["dY"]),
                   w.act, with_bias=w.bias)
    for k in ("dX", "dW1", "dW2") + (("db1",) if w.bias else ()):
        G.assert_parity(bo[k], rb[k], k)
    if w.has_attn:
        assert sp["qkv"] > 1, sp
        ao = G.run_attn_fwd(plan, inp)
        ra = L.attnproj_fwd(f64(inp["X"]), f64(inp["Wqkv"]), None, f64(inp["C"]), f64(inp["Wo"]))
        G.assert_parity(ao["QKV"], ra["QKV"], "QKV")
        G.assert_parity(ao["Z"], ra["Z"], "attn Z")
    for kw in (dict(n_row_slices=1, n_col_slices=1), dict(serialize=True), dict(tile="128x128")):
        p2 = T.plan_for(w, **kw)
        assert p2.info.splits() == sp, kw
        o2 = G.run_mlp_fwd(p2, inp)
        assert torch.equal(o2["Z"], out["Z"]) and torch.equal(o2["U"], out["U"]), kw
        b2 = G.run_mlp_bwd(p2, inp, with_bias=w.bias)
        for k in ("dX", "dW1", "dW2") + (("db1",) if w.bias else ()):
            assert torch.equal(b2[k], bo[k]), (kw, k)
        if w.has_attn:
            a2 = G.run_attn_fwd(p2, inp)
            assert torch.equal(a2["QKV"], ao["QKV"]) and torch.equal(a2["Z"], ao["Z"]), kw


def test_empty_batch():
    w = synth.custom("empty", 904, tokens=0, hidden=64, ffn=64, tp=1, act="gelu", bias=True, row_slices=2,
                     col_slices=2, backward=True)
    plan = T.plan_for(w)
    inp = synth.make_inputs(w)
    out = G.run_mlp_fwd(plan, inp)
    assert out["Z"].numel() == 0
    nan = lambda *s: torch.full(s, float("nan"), dtype=torch.float32, device="cuda")
    res = G.run_mlp_bwd(plan, inp, with_bias=True, init=(nan(64, 64), nan(64, 64), nan(64)))
    for k in ("dW1", "dW2", "db1"):
        assert torch.count_nonzero(res[k]) == 0 and not torch.isnan(res[k]).any(), k


def test_one_row_slices():
    w = synth.custom("one_row", 905, tokens=8, hidden=64, ffn=128, tp=2, act="swiglu", bias=False,
                     row_slices=8, col_slices=4, backward=True)
    inp = synth.make_inputs(w)
    plan = T.plan_for(w)
    out = G.run_mlp_fwd(plan, inp)
    G.assert_parity(out["Z"], G.oracle_mlp_fwd(inp, w.act)["Z"], "Z")
    assert torch.equal(out["Zh"], out["Z"])


# ------------------------------------------------------------------- full-size workloads, sampled
@pytest.mark.parametrize("key", ["gpt3_2.7b_mlp", "llama2_7b_mlp"])
def test_full_forward_workload(key):
    w = synth.WORKLOADS[key]
    _print_case("full_fwd", key=key)
    inp = synth.make_inputs(w)
    plan = T.plan_for(w)
    out = G.run_mlp_fwd(plan, inp)
    assert torch.equal(out["Zh"], out["Z"])
    rows = G.sample_rows(w.tokens, w.row_slices)
    ref = G.oracle_mlp_fwd(inp, w.act, rows=rows)
    G.assert_parity(out["Z"].cpu()[rows], ref["Z"], "Z rows")
    G.assert_parity(out["U"].cpu()[rows], ref["U"], "U rows")
    one = G.run_mlp_fwd(T.plan_for(w, n_row_slices=1, n_col_slices=1), inp, save_u=False, handoff=False)
    assert torch.equal(one["Z"], out["Z"])


@pytest.mark.parametrize("key", ["llama2_13b_layer", "llama3_70b_layer"])
def test_full_layer_workload(key):
    w = synth.WORKLOADS[key]
    _print_case("full_layer", key=key)
    inp = synth.make_inputs(w)
    plan = T.plan_for(w)
    rows = G.sample_rows(w.tokens, w.row_slices, per_slice=max(4, 32 // w.row_slices))
    # forward
    fo = G.run_mlp_fwd(plan, inp)
    ref = G.oracle_mlp_fwd(inp, w.act, rows=rows)
    G.assert_parity(fo["Z"].cpu()[rows], ref["Z"], "mlp Z rows")
    assert torch.equal(fo["Zh"], fo["Z"])
    del fo
    ao = G.run_attn_fwd(plan, inp)
    ra = L.attnproj_fwd(f64(inp["X"][rows]), f64(inp["Wqkv"]), None, f64(inp["C"][rows]), f64(inp["Wo"]))
    G.assert_parity(ao["QKV"].cpu()[rows], ra["QKV"], "QKV rows")
    G.assert_parity(ao["Z"].cpu()[rows], ra["Z"], "attn Z rows")
    assert torch.equal(ao["Zh"], ao["Z"])
    del ao
    # MLP backward: dX on sampled rows; weight gradients on sampled FFN columns (a column subset of
    # the shard is itself a shard, so the oracle runs on it with all tokens)
    bo = G.run_mlp_bwd(plan, inp, with_bias=False)
    assert torch.equal(bo["dXh"], bo["dX"])
    rb = L.mlp_bwd(f64(inp["X_mlp"][rows]), f64(inp["W1"]), f64(inp["W2"]), f64(inp["U_saved"][rows]),
                   f64(inp["dY"][rows]), w.act)
    G.assert_parity(bo["dX"].cpu()[rows], rb["dX"], "dX rows")
    Fp = w.ffn_shard
    J = G.sample_cols(Fp, 32)
    rows1 = np.concatenate([J, Fp + J])
    rj = L.mlp_bwd(f64(inp["X_mlp"]), f64(inp["W1"][rows1]), f64(inp["W2"][:, J]),
                   f64(inp["U_saved"][:, rows1]), f64(inp["dY"]), w.act)
    G.assert_parity(bo["dW1"].cpu()[rows1], rj["dW1"], "dW1 rows")
    G.assert_parity(bo["dW2"].cpu()[:, J], rj["dW2"], "dW2 cols")
    del bo
    # attention-projection backward
    go = G.run_attn_bwd(plan, inp, with_bias=False)
    assert torch.equal(go["dXh"], go["dX"])
    rg = L.attnproj_bwd(f64(inp["X"][rows]), f64(inp["Wqkv"]), f64(inp["dQKV"][rows]), f64(inp["C"][rows]),
                        f64(inp["Wo"]), f64(inp["dY_attn"][rows]))
    G.assert_parity(go["dX"].cpu()[rows], rg["dX"], "attn dX rows")
    G.assert_parity(go["dC"].cpu()[rows], rg["dC"], "dC rows")
    # weight gradients on sampled output rows: the oracle on that subset of the projections
    Jq = G.sample_cols(w.qkv_width, 32)
    Jh = G.sample_cols(w.hidden, 32)
    rs = L.attnproj_bwd(f64(inp["X"]), f64(inp["Wqkv"][Jq]), f64(inp["dQKV"][:, Jq]), f64(inp["C"]),
                        f64(inp["Wo"][Jh]), f64(inp["dY_attn"][:, Jh]))
    G.assert_parity(go["dWqkv"].cpu()[Jq], rs["dWqkv"], "dWqkv rows")
    G.assert_parity(go["dWo"].cpu()[Jh], rs["dWo"], "dWo rows")


@pytest.mark.parametrize("copy_blit", [False, True])
def test_handoff_complete_when_caller_stream_passes(copy_blit):
    """Work queued on the caller's stream after the call sees the finished hand-off copy (no
    device-wide synchronization in between)."""
    w = synth.WORKLOADS["gpt3_2.7b_mlp"]
    _print_case("join", key=w.key, copy_blit=copy_blit)
    inp = synth.make_inputs(w)
    plan = T.plan_for(w, copy_blit=copy_blit)
    X, W1, b1, W2 = (G.dev(inp[k]) for k in ("X_mlp", "W1", "b1", "W2"))
    i = plan.info
    Z = torch.empty((i.tokens, i.hidden), dtype=torch.bfloat16, device="cuda")
    Zh = torch.empty_like(Z)
    for rep in range(3):
        Zh.fill_(float("nan"))
        plan.mlp_fwd(X, W1, b1, W2, Z, None, Zh)
        snap = Zh.clone()          # queued on the caller stream right behind the call
        torch.cuda.synchronize()
        assert torch.equal(snap, Z), f"rep {rep}: hand-off not complete at the join"


ATTN_C2 = synth.custom("attn_c2", 913, tokens=520, hidden=272, ffn=64, tp=2, act="gelu", bias=False,
                       row_slices=2, col_slices=2, heads=6, kv_heads=2, head_dim=40, backward=True)


@pytest.mark.parametrize("w", [SMALL_GELU, SMALL_SWIGLU, ATTN_C2], ids=lambda w: w.key)
def test_handoff_whole_row_slices(w):
    """Whole-row hand-off (one contiguous copy per row slice after its last column piece) moves
    the same bytes: every output and hand-off buffer equals the per-piece run bit for bit, and
    work queued on the caller's stream right after the call sees the finished copies."""
    _print_case("handoff_rows", key=w.key)
    inp = synth.make_inputs(w)
    rows = T.plan_for(w, handoff_rows=True)
    pieces = T.plan_for(w)
    assert rows.info.n_col_slices > 1
    a, b = G.run_mlp_fwd(rows, inp, sync=False), None
    snap = a["Zh"].clone()
    torch.cuda.synchronize()
    b = G.run_mlp_fwd(pieces, inp)
    for k in ("Z", "U", "Zh"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(snap, a["Z"])
    if w.backward:
        a = G.run_mlp_bwd(rows, inp, with_bias=w.bias)
        b = G.run_mlp_bwd(pieces, inp, with_bias=w.bias)
        for k in ("dX", "dXh", "dW1", "dW2", "db1"):
            if a[k] is not None:
                assert torch.equal(a[k], b[k]), k
        assert torch.equal(a["dXh"], a["dX"])
    if w.has_attn:
        a = G.run_attn_fwd(rows, inp)
        b = G.run_attn_fwd(pieces, inp)
        for k in ("QKV", "Z", "Zh"):
            assert torch.equal(a[k], b[k]), k
        a = G.run_attn_bwd(rows, inp, with_bias=True)
        b = G.run_attn_bwd(pieces, inp, with_bias=True)
        for k in ("dX", "dXh", "dC", "dWqkv", "dWo", "dbqkv"):
            assert torch.equal(a[k], b[k]), k
    src = torch.randn(w.tokens, w.hidden, device="cuda").to(torch.bfloat16)
    dst = torch.zeros_like(src)
    rows.handoff_copy(src, dst)
    snap = dst.clone()
    torch.cuda.synchronize()
    assert torch.equal(snap, src)


@pytest.mark.parametrize("streams,rows", [(1, False), (2, False), (2, True)])
def test_pipelined_chain_matches_joined(streams, rows):
    """Four chained MLP calls, each reading the previous call's hand-off buffer as its input: the
    pipelined mode (per-slice waits instead of a full join) gives bitwise the same results."""
    w = synth.custom("chain", 906, tokens=1024, hidden=512, ffn=2048, tp=2, act="gelu", bias=True,
                     row_slices=4, col_slices=2)
    _print_case("pipeline", key=w.key, streams=streams, rows=rows)
    inp = synth.make_inputs(w)
    X0, W1, b1, W2 = (G.dev(inp[k]) for k in ("X_mlp", "W1", "b1", "W2"))

    def chain(plan, pipelined):
        i = plan.info
        Zs = [torch.empty((i.tokens, i.hidden), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
        Hs = [torch.full((i.tokens, i.hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
              for _ in range(4)]
        x = X0
        for n in range(4):
            plan.mlp_fwd(x, W1, b1, W2, Zs[n], None, Hs[n])
            x = Hs[n]
        if pipelined:
            plan.handoff_wait()
        torch.cuda.synchronize()
        return Hs

    ref = chain(T.plan_for(w), False)
    got = chain(T.plan_for(w, pipeline=True, n_streams=streams, handoff_rows=rows), True)
    for n in range(4):
        assert torch.equal(got[n], ref[n]), f"layer {n}"
    r1 = G.oracle_mlp_fwd(inp, w.act)
    G.assert_parity(ref[0], r1["Z"], "first layer")


def test_handoff_copy_only():
    w = synth.WORKLOADS["llama2_7b_mlp"]
    plan = T.plan_for(w)
    src = torch.randn(w.tokens, w.hidden, device="cuda").to(torch.bfloat16)
    dst = torch.zeros_like(src)
    plan.handoff_copy(src, dst)
    snap = dst.clone()
    torch.cuda.synchronize()
    assert torch.equal(snap, src)


def test_tracing_changes_no_result_and_times_every_launch():
    w = SMALL_SWIGLU
    inp = synth.make_inputs(w)
    plan = T.plan_for(w)
    base = G.run_mlp_fwd(plan, inp)
    plan.trace(True)
    out = G.run_mlp_fwd(plan, inp)
    recs = plan.trace_read()
    plan.trace(False)
    assert torch.equal(out["Z"], base["Z"]) and torch.equal(out["Zh"], base["Zh"])
    gemms = [r for r in recs if r["kind"] == "gemm"]
    copies = [r for r in recs if r["kind"] == "copy"]
    assert len(gemms) == w.row_slices * (1 + w.col_slices)
    assert len(copies) >= w.row_slices * w.col_slices
    assert all(r["end_ms"] > r["start_ms"] >= 0 for r in gemms)
    fl = w.gemm_flops()
    assert sum(r["flops"] for r in gemms) == pytest.approx(fl["mlp_up"] + fl["mlp_down"])


def _chain_step(plan, w, d, x, o, g, dy_mlp):
    """One layer step as the benchmark chains them: the attention projections read `x`, the MLP reads
    their hand-off, the MLP backward takes `dy_mlp`, the attention backward the MLP's dX hand-off."""
    if w.has_attn:
        plan.attnproj_fwd(x, d["Wqkv"], None, o["QKV"], d["C"], d["Wo"], o["Za"], o["Zah"])
        x_mlp = o["Zah"]
    else:
        x_mlp = x
    plan.mlp_fwd(x_mlp, d["W1"], d.get("b1"), d["W2"], o["Z"], o["U"], o["Zh"])
    if w.backward:
        plan.mlp_bwd(x_mlp, d["W1"], d["W2"], d["U_saved"], dy_mlp, o["dX"], g["dW1"], g["dW2"],
                     db1=g.get("db1"), dX_handoff=o["dXh"])
        if w.has_attn:
            plan.attnproj_bwd(x, d["Wqkv"], d["dQKV"], d["C"], d["Wo"], o["dXh"], o["dXa"], o["dC"], g["dWqkv"],
                              g["dWo"], dX_handoff=o["dXah"])


def _chain_buffers(w, i):
    e = lambda *s, dt=torch.bfloat16: torch.full(s, float("nan"), dtype=dt, device="cuda")
    o = {"Z": e(i.tokens, i.hidden), "Zh": e(i.tokens, i.hidden), "U": e(i.tokens, i.n1)}
    if w.has_attn:
        o.update(QKV=e(i.tokens, i.qkv_width), Za=e(i.tokens, i.hidden), Zah=e(i.tokens, i.hidden))
    g = {}
    if w.backward:
        o.update(dX=e(i.tokens, i.hidden), dXh=e(i.tokens, i.hidden))
        g = {"dW1": e(i.n1, i.hidden, dt=torch.float32), "dW2": e(i.hidden, i.ffn_shard, dt=torch.float32)}
        if w.bias:
            g["db1"] = e(i.n1, dt=torch.float32)
        if w.has_attn:
            o.update(dXa=e(i.tokens, i.hidden), dXah=e(i.tokens, i.hidden), dC=e(i.tokens, i.ctx_width))
            g.update(dWqkv=e(i.qkv_width, i.hidden, dt=torch.float32), dWo=e(i.hidden, i.ctx_width, dt=torch.float32))
    return o, g


@pytest.mark.parametrize("key", ["llama2_7b_mlp", "llama3_70b_layer"])
def test_benchmark_mode_full_size(key):
    """The plan flags the benchmark times (pipelined hand-off, whole-row copies, default streams) over
    two chained layer steps at full size, each step reading the previous step's hand-off: every
    output and hand-off buffer equals bit for bit the same steps run with joined calls (whose outputs
    the full-size tests above check against the oracle), and the first step's MLP output on sampled
    rows of every row slice matches the oracle."""
    w = synth.WORKLOADS[key]
    _print_case("bench_mode", key=key)
    inp = synth.make_inputs(w)
    d = {k: v.to("cuda").contiguous() for k, v in inp.items()}
    bench_plan = T.plan_for(w, pipeline=True, handoff_rows=True)
    joined = T.plan_for(w)
    assert bench_plan.info.n_col_slices == w.col_slices
    x0 = d["X"] if w.has_attn else d["X_mlp"]
    dy = d.get("dY")
    outs = {}
    for name, plan in (("bench", bench_plan), ("joined", joined)):
        o1, g1 = _chain_buffers(w, plan.info)
        o2, g2 = _chain_buffers(w, plan.info)
        _chain_step(plan, w, d, x0, o1, g1, dy)
        _chain_step(plan, w, d, o1["Zh"], o2, g2, dy)
        plan.handoff_wait()
        torch.cuda.synchronize()
        outs[name] = (o1, g1, o2, g2)
    for a, b in zip(outs["bench"], outs["joined"]):
        for k in a:
            assert torch.equal(a[k], b[k]), k
    o1 = outs["bench"][0]
    for k in ("Zh", "dXh", "Zah", "dXah"):
        if k in o1:
            assert torch.equal(o1[k], o1[k[:-1]]), k
    if not w.has_attn:
        rows = G.sample_rows(w.tokens, w.row_slices, per_slice=max(4, 32 // w.row_slices))
        ref = G.oracle_mlp_fwd(inp, w.act, rows=rows)
        G.assert_parity(o1["Z"].cpu()[rows], ref["Z"], "Z rows")
    bench_plan.close()
    joined.close()


# Pipelined calls whose caller passes another set of worker and copy streams each time: a call's
# waits for earlier calls' copies must hold whatever streams those copies ran on (a wait for one
# copy record is taken to cover earlier ones only within one call and one stream), and the first
# row slice after a call that ran products over all tokens behind its copies waits for all of them.
STREAMS_LAYER = synth.custom("streams_layer", 915, tokens=2048, hidden=512, ffn=1024, tp=2, act="swiglu",
                             bias=False, row_slices=4, col_slices=2, heads=8, kv_heads=2, head_dim=64,
                             backward=True)


@pytest.mark.parametrize("streams", [1, 2])
def test_pipelined_calls_with_changing_streams(streams):
    w = STREAMS_LAYER
    _print_case("changing_streams", key=w.key, streams=streams)
    inp = synth.make_inputs(w)
    d = {k: v.to("cuda").contiguous() for k, v in inp.items()}
    plan = T.plan_for(w, pipeline=True, handoff_rows=True, n_streams=streams, n_copy_streams=2)
    joined = T.plan_for(w)
    i = plan.info
    assert i.n_streams == streams and i.n_copy_streams == 2
    sets = [T.Streams.new(i.n_streams if i.n_streams > 1 else 0, 2) for _ in range(3)]
    calls = [0]

    def rotate():
        plan.streams = sets[calls[0] % len(sets)]
        calls[0] += 1

    def step(pl, x, o, g, turn):
        if turn: rotate()
        pl.attnproj_fwd(x, d["Wqkv"], None, o["QKV"], d["C"], d["Wo"], o["Za"], o["Zah"])
        if turn: rotate()
        pl.mlp_fwd(o["Zah"], d["W1"], None, d["W2"], o["Z"], o["U"], o["Zh"])
        if turn: rotate()
        pl.mlp_bwd(o["Zah"], d["W1"], d["W2"], d["U_saved"], o["Zh"], o["dX"], g["dW1"], g["dW2"],
                   dX_handoff=o["dXh"])
        if turn: rotate()
        pl.attnproj_bwd(x, d["Wqkv"], d["dQKV"], d["C"], d["Wo"], o["dXh"], o["dXa"], o["dC"], g["dWqkv"],
                        g["dWo"], dX_handoff=o["dXah"])

    outs = {}
    for name, pl, turn in (("pipelined", plan, True), ("joined", joined, False)):
        bufs = [_chain_buffers(w, pl.info) for _ in range(3)]
        x = d["X"]
        for o, g in bufs:
            step(pl, x, o, g, turn)
            x = o["dXah"]
        if turn:
            for s in sets:
                plan.streams = s
                plan.handoff_wait()
        torch.cuda.synchronize()
        outs[name] = bufs
    for n, ((o1, g1), (o2, g2)) in enumerate(zip(outs["pipelined"], outs["joined"])):
        for k in o1:
            assert torch.equal(o1[k], o2[k]), (n, k)
        for k in g1:
            assert torch.equal(g1[k], g2[k]), (n, k)
    o = outs["joined"][0][0]
    for k in ("Zh", "dXh", "Zah", "dXah"):
        assert torch.equal(o[k], o[k[:-1]]), k
    plan.close()
    joined.close()


# Producers over groups of row slices: the up-projection and dH take the whole batch's k split,
# so every group size gives the same bits; the grouped plan also matches the oracle.
GROUPS = synth.custom("groups", 912, tokens=2048, hidden=512, ffn=1536, tp=2, act="swiglu", bias=True,
                      row_slices=8, col_slices=2, backward=True)


@pytest.mark.parametrize("group,streams", [(2, 1), (8, 1), (2, 2)])
def test_producer_groups_keep_the_bits(group, streams):
    """Groups of one, two and all eight row slices, on one worker stream and on two (a group's
    producer then runs on the first slice's worker and the other slices wait for it)."""
    w = GROUPS
    _print_case("producer_groups", key=w.key, group=group, streams=streams)
    inp = synth.make_inputs(w)
    base = T.plan_for(w, up_group=1, dh_group=1, handoff_rows=True)
    grouped = T.plan_for(w, up_group=group, dh_group=group, handoff_rows=True, n_streams=streams)
    assert grouped.info.n_streams == streams
    assert grouped.info.up_group_slices == group and grouped.info.dh_group_slices == group
    assert grouped.info.splits() == base.info.splits()
    fa, fb = G.run_mlp_fwd(base, inp), G.run_mlp_fwd(grouped, inp)
    for k in ("Z", "U", "Zh"):
        assert torch.equal(fa[k], fb[k]), k
    ba, bb = G.run_mlp_bwd(base, inp, with_bias=True), G.run_mlp_bwd(grouped, inp, with_bias=True)
    for k in ("dX", "dXh", "dW1", "dW2", "db1"):
        assert torch.equal(ba[k], bb[k]), k
    ref = G.oracle_mlp_fwd(inp, w.act)
    G.assert_parity(fb["Z"], ref["Z"], "Z")
    rb = L.mlp_bwd(f64(inp["X_mlp"]), f64(inp["W1"]), f64(inp["W2"]), f64(inp["U_saved"]), f64(inp["dY"]),
                   w.act, with_bias=True)
    for k in ("dX", "dW1", "dW2", "db1"):
        G.assert_parity(bb[k], rb[k], k)
    base.close()
    grouped.close()
