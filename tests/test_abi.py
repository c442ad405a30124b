"""CPU tests of the C ABI: the library loads, exports every declared symbol, validates plans and
arguments before any GPU work, and its slice geometry equals the oracle's bit for bit."""
import ctypes
import os
import re

import pytest

from comm_overlap_amd import synth
from oracle import plan as OP

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
T = pytest.importorskip("comm_overlap_amd.tpslice", reason="libtpslice.so not built")


def declared_symbols():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", fn)).read()
            names |= set(re.findall(r"TPSLICE_API\s+[\w\s\*]+?\b(tpslice_\w+)\s*\(", txt))
    return names


def test_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) >= 11
    lib = ctypes.CDLL(T.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(T.EXPORTS) == names


@pytest.mark.parametrize("key", list(synth.WORKLOADS))
def test_geometry_matches_oracle(key):
    w = synth.WORKLOADS[key]
    p = T.plan_for(w)
    i = p.info
    assert (i.tokens, i.hidden, i.ffn_shard, i.n1) == (w.tokens, w.hidden, w.ffn_shard, w.n1)
    if w.has_attn:
        assert (i.qkv_width, i.ctx_width, i.q_heads, i.kv_heads) == (
            w.qkv_width, w.ctx_width, w.q_heads_shard, w.kv_heads_shard)
    pieces = [p.piece(k) for k in range(w.row_slices * w.col_slices)]
    assert pieces == OP.handoff_pieces(w.tokens, w.hidden, w.row_slices, w.col_slices)
    with pytest.raises(T.TpsliceError):
        p.piece(w.row_slices * w.col_slices)


@pytest.mark.parametrize("M,h,r,c", [(24, 40, 3, 5), (8, 64, 8, 8), (1024, 1024, 16, 4), (0, 8, 3, 1)])
def test_geometry_small(M, h, r, c):
    p = T.Plan(T.Config(tokens=M, hidden=h, ffn=64, n_row_slices=r, n_col_slices=c))
    got = [p.piece(k) for k in range(r * c)]
    if M == 0:
        assert all(g[0] == g[1] == 0 for g in got)
    else:
        assert got == OP.handoff_pieces(M, h, r, c)


@pytest.mark.parametrize("kw,code", [
    (dict(tokens=100, hidden=64, ffn=64, n_row_slices=3), T.ERR_SHAPE),
    (dict(tokens=64, hidden=60, ffn=64), T.ERR_SHAPE),
    (dict(tokens=64, hidden=64, ffn=100, tp_size=2), T.ERR_SHAPE),      # shard 50 not a multiple of 8
    (dict(tokens=64, hidden=64, ffn=64, tp_size=3), T.ERR_SHAPE),
    (dict(tokens=64, hidden=64, ffn=64, n_col_slices=3), T.ERR_SHAPE),
    (dict(tokens=64, hidden=64, ffn=64, n_col_slices=16), T.ERR_SHAPE),  # 4 columns per slice
    (dict(tokens=64, hidden=64, ffn=64, act="relu"), T.ERR_INVALID),
    (dict(tokens=64, hidden=64, ffn=64, n_heads=6, n_kv_heads=2, head_dim=12), T.ERR_SHAPE),
    (dict(tokens=64, hidden=64, ffn=64, n_heads=6, n_kv_heads=0, head_dim=16), T.ERR_SHAPE),
    (dict(tokens=64, hidden=64, ffn=64, n_streams=99), T.ERR_SHAPE),
    (dict(tokens=1 << 20, hidden=4096, ffn=4096), T.ERR_SHAPE),          # 8 GiB operand
    (dict(tokens=64, hidden=64, ffn=64, n_row_slices=-1), T.ERR_SHAPE),
    (dict(tokens=64, hidden=64, ffn=64, n_row_slices=0, handoff_gbps=-1.0), T.ERR_SHAPE),
    (dict(tokens=64, hidden=64, ffn=64, n_row_slices=0, handoff_gbps=float("nan")), T.ERR_SHAPE),
])
def test_plan_rejects(kw, code):
    with pytest.raises(T.TpsliceError) as e:
        T.Plan(T.Config(**kw))
    assert e.value.code == code


def test_gqa_kv_heads_below_tp():
    p = T.plan_for(synth.WORKLOADS["llama3_70b_layer"])
    assert (p.info.q_heads, p.info.kv_heads, p.info.qkv_width) == (8, 1, 1280)


def test_workspace_sizes():
    w = synth.WORKLOADS["llama3_70b_layer"]
    p = T.plan_for(w)
    M, Fp, N1 = w.tokens, w.ffn_shard, w.n1
    assert p.workspace_size(T.OP_MLP_FWD) == M * Fp * 2
    assert p.workspace_size(T.OP_MLP_BWD) >= M * N1 * 2 + M * Fp * 2
    assert p.workspace_size(T.OP_ATTNPROJ_FWD) >= 0
    with pytest.raises(T.TpsliceError):
        p.workspace_size(7)


def _fake(addr):
    return ctypes.c_void_p(addr)


def test_argument_errors_before_any_gpu_work():
    """Null, misaligned, workspace and plan errors come back before anything touches the GPU (the
    pointers below are never dereferenced)."""
    lib = T.lib
    p = T.Plan(T.Config(tokens=64, hidden=64, ffn=64, n_row_slices=2))
    A = _fake(0x100000)
    ws_need = p.workspace_size(T.OP_MLP_FWD)
    # NULL required pointer
    assert lib.tpslice_mlp_fwd(p._h, None, A, None, A, A, None, None, A, ws_need, None) == T.ERR_INVALID
    assert b"X is NULL" in lib.tpslice_last_error()
    # misaligned pointer
    assert lib.tpslice_mlp_fwd(p._h, _fake(0x100002), A, None, A, A, None, None, A, ws_need,
                               None) == T.ERR_INVALID
    # workspace too small / missing / misaligned
    assert lib.tpslice_mlp_fwd(p._h, A, A, None, A, A, None, None, A, ws_need - 1, None) == T.ERR_WORKSPACE
    assert lib.tpslice_mlp_fwd(p._h, A, A, None, A, A, None, None, None, 0, None) == T.ERR_WORKSPACE
    assert lib.tpslice_mlp_fwd(p._h, A, A, None, A, A, None, None, _fake(0x100010), ws_need,
                               None) == T.ERR_WORKSPACE
    # invalid plan handle
    assert lib.tpslice_mlp_fwd(None, A, A, None, A, A, None, None, A, ws_need, None) == T.ERR_INVALID
    # attention entry points on a plan without heads
    assert lib.tpslice_attnproj_fwd(p._h, A, A, None, A, A, A, A, None, None, 0, None) == T.ERR_UNSUPPORTED
    assert lib.tpslice_attnproj_bwd(p._h, A, A, A, A, A, A, A, None, A, A, None, A, 0, None, 0,
                                    None) == T.ERR_UNSUPPORTED
    # bad accumulate flag
    wsb = p.workspace_size(T.OP_MLP_BWD)
    assert lib.tpslice_mlp_bwd(p._h, A, A, A, A, A, A, None, A, None, A, 2, A, wsb, None) == T.ERR_INVALID
    assert lib.tpslice_error_string(T.ERR_WORKSPACE) == b"workspace too small or misaligned"
    p.close()
    p.close()  # idempotent in the binding


def test_serialize_plan_uses_one_stream():
    p = T.Plan(T.Config(tokens=64, hidden=64, ffn=64, n_row_slices=4, serialize=True))
    assert (p.info.n_streams, p.info.n_copy_streams) == (1, 1)


def test_pipeline_flag_and_handoff_wait_without_gpu_work():
    p = T.Plan(T.Config(tokens=64, hidden=64, ffn=64, n_row_slices=2, pipeline=True))
    p.handoff_wait.__func__  # bound
    # before any call there is nothing to wait for: returns OK without touching the GPU
    assert T.lib.tpslice_handoff_wait(p._h, None) == T.OK
    assert T.lib.tpslice_handoff_copy(None, None, None, None) == T.ERR_INVALID


def test_plan_tile_flags():
    import ctypes
    d = T.Config(tokens=64, hidden=64, ffn=64).desc()
    d.flags = 11 << T.F_TILE_SHIFT  # ids run 0..10
    h = ctypes.c_void_p()
    assert T.lib.tpslice_plan(ctypes.byref(d), ctypes.byref(h)) == T.ERR_INVALID
    assert b"tile id" in T.lib.tpslice_last_error()
    for tile in T.TILES:
        T.Plan(T.Config(tokens=64, hidden=64, ffn=64, tile=tile)).close()


LARGE = ["gpt3_2.7b_mlp", "llama2_7b_mlp", "llama2_13b_layer", "llama3_70b_layer"]


@pytest.mark.parametrize("key", ["tiny_gpt_mlp"] + LARGE)
@pytest.mark.parametrize("pipeline", [False, True])
@pytest.mark.parametrize("gbps", [0.0, 100.0, 25.0])
def test_automatic_slice_counts_are_valid(key, pipeline, gbps):
    w = synth.WORKLOADS[key]
    p = T.plan_for(w, n_row_slices=0, n_col_slices=0, pipeline=pipeline, handoff_gbps=gbps)
    r, c = p.info.n_row_slices, p.info.n_col_slices
    assert r in (1, 2, 4, 8, 16) and w.tokens % r == 0
    assert c in (1, 2, 4) and w.hidden % c == 0 and (w.hidden // c) % 8 == 0
    assert p.info.rows_per_slice * r == w.tokens and p.info.handoff_cols * c == w.hidden
    assert p.info.predicted_forward_us > 0
    # the choice is the model's best over the candidates (fewer pieces within 2%)
    best = min(T.plan_for(w, n_row_slices=rr, n_col_slices=cc, pipeline=pipeline, handoff_gbps=gbps)
               .info.predicted_forward_us
               for rr in (1, 2, 4, 8, 16) if w.tokens % rr == 0
               for cc in (1, 2, 4) if w.hidden % cc == 0 and (w.hidden // cc) % 8 == 0)
    assert p.info.predicted_forward_us <= best * 1.02 + 1e-9


def test_slow_handoff_slices_a_small_layer():
    """The slicing the GPU test of automatic slice counts runs (2048 tokens, h 1024, F 4096, GeLU):
    with a 25 GB/s hand-off the model slices it, with the local DMA copy it does not (pins the
    chooser's own worker-stream count, which must use the plan's product widths)."""
    w = synth.custom("auto_slices", 909, tokens=2048, hidden=1024, ffn=4096, tp=1, act="gelu", bias=True,
                     row_slices=1, col_slices=1)
    slow = T.plan_for(w, n_row_slices=0, n_col_slices=0, handoff_gbps=25.0)
    assert slow.info.n_row_slices * slow.info.n_col_slices > 1
    fast = T.plan_for(w, n_row_slices=0, n_col_slices=0)
    assert fast.info.n_row_slices * fast.info.n_col_slices >= 1


def test_whole_row_handoff_runs_one_product_per_row_slice():
    """With whole-row hand-off the chooser and the plan model one product of h columns per row
    slice: the prediction equals that of the same plan with one column slice."""
    w = synth.WORKLOADS["llama3_70b_layer"]
    rows = T.plan_for(w, handoff_rows=True, n_streams=2)
    one = T.plan_for(w, n_col_slices=1, n_streams=2)
    assert rows.info.n_col_slices == 2
    assert rows.info.predicted_forward_us == pytest.approx(one.info.predicted_forward_us, rel=1e-12)


@pytest.mark.parametrize("key", LARGE)
def test_dh_groups_divide_the_row_slices_and_keep_the_split(key):
    """dH runs over groups of row slices: the group size divides r, and the k split (the whole
    batch's) is the same for every slicing, so that sliced and unsliced backward passes keep the
    same bits. On the 70B shard a 2048-row slice's dH fills 112 of 256 CUs: two row slices a group."""
    w = synth.WORKLOADS[key]
    base = T.plan_for(w, n_row_slices=1, n_col_slices=1).info
    assert base.dh_group_slices == 1
    for r in (1, 2, 4, 8):
        if w.tokens % r:
            continue
        i = T.plan_for(w, n_row_slices=r).info
        assert r % i.dh_group_slices == 0
        assert i.splits()["dh"] == base.splits()["dh"]
    if key == "llama3_70b_layer":
        assert T.plan_for(w).info.dh_group_slices == 2
    # a requested group size is kept; one that does not divide r, or is no power of two, is refused
    r = T.plan_for(w).info.n_row_slices
    assert T.plan_for(w, dh_group=r).info.dh_group_slices == r
    for bad in (2 * r, 3, -1):
        with pytest.raises(T.TpsliceError) as e:
            T.plan_for(w, dh_group=bad)
        assert e.value.code == T.ERR_INVALID


@pytest.mark.parametrize("key", LARGE)
def test_up_groups_divide_the_row_slices_and_keep_the_split(key):
    """The up-projection runs over groups of row slices: the group divides r, the k split (the whole
    batch's) is the same for every slicing, a plan with two worker streams keeps one row slice per
    up-projection, and a requested group is kept (or refused when it does not divide r)."""
    w = synth.WORKLOADS[key]
    base = T.plan_for(w, n_row_slices=1, n_col_slices=1).info
    assert base.up_group_slices == 1
    for r in (1, 2, 4, 8):
        if w.tokens % r:
            continue
        i = T.plan_for(w, n_row_slices=r).info
        assert r % i.up_group_slices == 0
        assert i.splits()["up"] == base.splits()["up"]
        if i.n_streams > 1:
            assert i.up_group_slices == 1
        assert T.plan_for(w, n_row_slices=r, n_streams=2).info.up_group_slices == 1
    r = T.plan_for(w).info.n_row_slices
    assert T.plan_for(w, up_group=r).info.up_group_slices == r
    with pytest.raises(T.TpsliceError) as e:
        T.plan_for(w, up_group=2 * r)
    assert e.value.code == T.ERR_INVALID
    if key == "llama3_70b_layer":  # 8 x 32 tiles of 256 x 224 per row slice; all 16384 rows: 1792 of 256 x 256
        assert T.plan_for(w).info.up_group_slices == 8


@pytest.mark.parametrize("key", sorted(synth.WORKLOADS))
def test_tail_splits_cover_the_last_rows_of_weight_gradients(key):
    """A split covers the whole product, or only a weight gradient's last rows (a tail split: the
    other rows, a multiple of 256, run unsplit). The choice depends on the product's shape only, so
    every slicing gets the same one; the tail's partial buffers are all the workspace holds for it."""
    w = synth.WORKLOADS[key]
    i = T.plan_for(w).info
    product_rows = {"dw1": i.n1, "dw2": i.hidden, "dwo": i.hidden, "dwqkv": i.qkv_width, "qkv": i.tokens,
                    "dc": i.tokens}
    sp, rows = i.splits(), i.split_rows()
    for k in T.PlanInfo.SPLIT_NAMES:
        assert (rows[k] == 0) == (sp[k] == 1), (k, sp[k], rows[k])
        if sp[k] > 1 and k in product_rows and rows[k] != product_rows[k]:
            assert k in ("dw1", "dw2", "dwo", "dwqkv"), k
            assert 0 < rows[k] < product_rows[k] and (product_rows[k] - rows[k]) % 256 == 0, (k, rows[k])
    for r in (1, 2, 4, 8):
        if w.tokens % r:
            continue
        j = T.plan_for(w, n_row_slices=r).info
        for k in ("dw1", "dw2", "dwo", "dwqkv"):
            assert (j.splits()[k], j.split_rows()[k]) == (sp[k], rows[k]), (r, k)
    expect = {"llama3_70b_layer": (2, 1024), "llama2_13b_layer": (4, 384)}
    if key in expect:
        # 70B dW1: 28 x 32 tiles = 3.5 rounds -> 24 tile rows unsplit, the last 4 split in two;
        # 13B dW1: 14 x 20 tiles -> 12 tile rows unsplit (one round), the last 384 rows split in four
        assert (sp["dw1"], rows["dw1"]) == expect[key]
        whole = sp["dw1"] * i.n1 * i.hidden * 4  # what a split of the whole product would need
        assert T.plan_for(w).workspace_size(T.OP_MLP_BWD) < whole


def test_given_slice_counts_are_kept():
    w = synth.WORKLOADS["llama3_70b_layer"]
    for gbps in (0.0, 25.0):
        p = T.plan_for(w, handoff_gbps=gbps)
        assert (p.info.n_row_slices, p.info.n_col_slices) == (w.row_slices, w.col_slices)
    # one count given, the other automatic
    p = T.plan_for(w, n_row_slices=4, n_col_slices=0)
    assert p.info.n_row_slices == 4 and p.info.n_col_slices in (1, 2, 4)


@pytest.mark.parametrize("streams", [1, 2])
@pytest.mark.parametrize("key", LARGE)
def test_slower_handoff_never_takes_fewer_row_slices_for_isolated_calls(key, streams):
    """Isolated calls expose the last row slice's hand-off, so while the products take longer than
    the copies, a slower hand-off is worth at least as many row slices, for a given number of worker
    streams (left open, the stream count follows the slice size, which can turn a finer slicing into
    the faster one at a faster hand-off). Once the copies take longer, slicing saves only the first
    slice's products, a fixed time that the rule's 2% margin for more pieces can outweigh."""
    w = synth.WORKLOADS[key]
    comp = T.plan_for(w, n_row_slices=1, n_col_slices=1, handoff_gbps=1e6, n_streams=streams).info.predicted_forward_us
    tensors = 2 if w.has_attn else 1
    rates = [g for g in (0.0, 400.0, 200.0, 100.0, 50.0)
             if g == 0.0 or w.tokens * w.hidden * 2 * tensors / (g * 1e3) <= comp]
    assert len(rates) >= 2
    rs = [T.plan_for(w, n_row_slices=0, n_col_slices=1, handoff_gbps=g, n_streams=streams).info.n_row_slices
          for g in rates]
    assert rs == sorted(rs), (rates, rs)


@pytest.mark.parametrize("key", LARGE)
def test_pipelined_chain_slices_to_hide_its_copy(key):
    """In a pipelined chain the next call's row slice 0 waits for this call's copy of row slice 0,
    so one row slice leaves its whole copy exposed: with the local DMA hand-off the model slices
    (the measured sweep: GPT-3 2.7B 1109-1124 TFLOP/s at r = 2 against 1059-1067 unsliced), and
    with a hand-off that costs nothing it keeps the products whole."""
    w = synth.WORKLOADS[key]
    p = T.plan_for(w, n_row_slices=0, n_col_slices=0, pipeline=True, handoff_rows=True)
    assert p.info.n_row_slices >= 2
    free = T.plan_for(w, n_row_slices=0, n_col_slices=0, pipeline=True, handoff_rows=True, handoff_gbps=1e6)
    assert free.info.n_row_slices <= p.info.n_row_slices
    if free.info.n_streams == 1:  # (two worker streams may slice for the products' own overlap)
        assert free.info.n_row_slices * free.info.n_col_slices == 1
    one = T.plan_for(w, n_row_slices=1, n_col_slices=1, pipeline=True, handoff_rows=True).info.predicted_forward_us
    one_free = T.plan_for(w, n_row_slices=1, n_col_slices=1, pipeline=True, handoff_rows=True,
                          handoff_gbps=1e6).info.predicted_forward_us
    assert one > one_free  # the exposed copy


def test_caller_worker_flag():
    """Worker 0 on the caller's stream: accepted with and without pipelining; nothing to wait for
    before the first call."""
    for pipeline in (False, True):
        p = T.Plan(T.Config(tokens=64, hidden=64, ffn=64, n_row_slices=2, n_streams=2, pipeline=pipeline,
                            caller_worker=True))
        assert p.info.n_streams == 2
        assert T.lib.tpslice_handoff_wait(p._h, None) == T.OK
        p.close()
    d = T.Config(tokens=64, hidden=64, ffn=64).desc()
    d.flags = 0x80  # an unknown bit next to it
    import ctypes
    h = ctypes.c_void_p()
    assert T.lib.tpslice_plan(ctypes.byref(d), ctypes.byref(h)) == T.ERR_INVALID


def test_handoff_rows_flag():
    """Whole-row hand-off is accepted with and without column slices and pipelining; the plan's
    slicing is unchanged by it."""
    for c in (1, 2):
        for pipeline in (False, True):
            p = T.Plan(T.Config(tokens=64, hidden=64, ffn=64, n_row_slices=2, n_col_slices=c, pipeline=pipeline,
                                handoff_rows=True))
            assert (p.info.n_row_slices, p.info.n_col_slices) == (2, c)
            p.close()
    assert T.F_HANDOFF_ROWS == 0x8


def test_attention_core_argument_errors():
    """The attention core (forward and backward) checks its plan, sizes, pointers and workspace
    before any GPU work (pointers never read)."""
    lib = T.lib
    A = _fake(0x100000)
    no_heads = T.Plan(T.Config(tokens=256, hidden=64, ffn=64))
    assert lib.tpslice_attn_core_fwd(no_heads._h, A, A, None, 128, None) == T.ERR_UNSUPPORTED
    d64 = T.Plan(T.Config(tokens=256, hidden=512, ffn=64, n_heads=4, n_kv_heads=2, head_dim=64))
    assert lib.tpslice_attn_core_fwd(d64._h, A, A, None, 128, None) == T.ERR_UNSUPPORTED
    assert b"head_dim 64" in lib.tpslice_last_error()
    p = T.Plan(T.Config(tokens=256, hidden=512, ffn=64, n_heads=4, n_kv_heads=2, head_dim=128))
    for bad in (0, -128, 64, 96, 192, 512):  # not a multiple of 128, or not dividing the 256 tokens
        assert lib.tpslice_attn_core_fwd(p._h, A, A, None, bad, None) == T.ERR_SHAPE, bad
    assert lib.tpslice_attn_core_fwd(p._h, None, A, None, 128, None) == T.ERR_INVALID
    assert lib.tpslice_attn_core_fwd(p._h, A, _fake(0x100008), None, 128, None) == T.ERR_INVALID
    assert lib.tpslice_attn_core_fwd(p._h, A, A, _fake(0x100004), 128, None) == T.ERR_INVALID
    assert lib.tpslice_attn_core_fwd(None, A, A, None, 128, None) == T.ERR_INVALID
    # backward: the workspace holds D per (token, query head) and, with grouped heads (4 query
    # heads over 2 key/value heads here), fp32 dK and dV partials of every query head
    need = p.workspace_size(T.OP_ATTN_CORE_BWD)
    assert need >= 256 * 4 * 4 + 2 * 4 * 256 * 128 * 4
    bwd = lib.tpslice_attn_core_bwd
    assert bwd(p._h, A, A, A, A, A, 128, A, need - 1, None) == T.ERR_WORKSPACE
    assert bwd(p._h, A, A, A, A, A, 128, None, 0, None) == T.ERR_WORKSPACE
    assert bwd(p._h, A, A, None, A, A, 128, A, need, None) == T.ERR_INVALID
    assert bwd(p._h, A, A, A, A, A, 96, A, need, None) == T.ERR_SHAPE
    assert bwd(d64._h, A, A, A, A, A, 128, A, need, None) == T.ERR_UNSUPPORTED
    ungrouped = T.Plan(T.Config(tokens=256, hidden=512, ffn=64, n_heads=4, n_kv_heads=4, head_dim=128))
    assert ungrouped.workspace_size(T.OP_ATTN_CORE_BWD) == 256 * 4 * 4  # D only


def test_bench_rejects_more_than_one_gpu():
    """bench.py measures one GPU; --gpus above 1 exits with a message before touching a GPU."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_static_scratch_entry_rejects_before_any_gpu_work():
    """The allocation-free forward checks its plan and the workspace size before it looks up the
    device array or queues anything (the pointers below are never dereferenced)."""
    lib = T.lib
    A = _fake(0x100000)
    assert lib.tpslice_mlp_fwd_static(None, A, A, None, A, A, None, None, None) == T.ERR_INVALID
    big = T.Plan(T.Config(tokens=8192, hidden=1024, ffn=8192, n_row_slices=2))
    assert big.workspace_size(T.OP_MLP_FWD) > T.STATIC_SCRATCH_BYTES
    assert lib.tpslice_mlp_fwd_static(big._h, A, A, None, A, A, None, None, None) == T.ERR_WORKSPACE
    assert b"static scratch" in lib.tpslice_last_error()
    big.close()
