"""A layer step of a joined (not pipelined) plan captured into a HIP graph: the QKV and output
projections, the MLP forward and backward and the projections' backward, with their hand-off
copies. Every replay, with eager work and synchronization between replays, gives the bits of the
same calls run eagerly (the copies become graph copy nodes; no call allocates, synchronizes or
clears memory)."""
import pytest
import torch

from comm_overlap_amd import synth
import gpu_cases as G

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from comm_overlap_amd import tpslice as T

LAYER = synth.custom("graph_layer", 960, tokens=1024, hidden=512, ffn=1024, tp=2, act="swiglu", bias=True,
                     row_slices=4, col_slices=2, heads=8, kv_heads=2, head_dim=64, backward=True)


def _outputs(i):
    bf, f32 = torch.bfloat16, torch.float32
    e = lambda *s, dt=bf: torch.empty(*s, dtype=dt, device="cuda")
    return dict(QKV=e(i.tokens, i.qkv_width), Za=e(i.tokens, i.hidden), Zah=e(i.tokens, i.hidden),
                Z=e(i.tokens, i.hidden), Zh=e(i.tokens, i.hidden), U=e(i.tokens, i.n1), dX=e(i.tokens, i.hidden),
                dXh=e(i.tokens, i.hidden), dW1=e(i.n1, i.hidden, dt=f32), dW2=e(i.hidden, i.ffn_shard, dt=f32),
                db1=e(i.n1, dt=f32), dXa=e(i.tokens, i.hidden), dXah=e(i.tokens, i.hidden),
                dC=e(i.tokens, i.ctx_width), dWqkv=e(i.qkv_width, i.hidden, dt=f32),
                dWo=e(i.hidden, i.ctx_width, dt=f32), dbqkv=e(i.qkv_width, dt=f32))


def _step(p, d, o):
    p.attnproj_fwd(d["X"], d["Wqkv"], None, o["QKV"], d["C"], d["Wo"], o["Za"], o["Zah"])
    p.mlp_fwd(o["Zah"], d["W1"], d["b1"], d["W2"], o["Z"], o["U"], o["Zh"])
    p.mlp_bwd(o["Zah"], d["W1"], d["W2"], o["U"], d["dY"], o["dX"], o["dW1"], o["dW2"], db1=o["db1"],
              dX_handoff=o["dXh"])
    p.attnproj_bwd(d["X"], d["Wqkv"], d["dQKV"], d["C"], d["Wo"], o["dXh"], o["dXa"], o["dC"], o["dWqkv"],
                   o["dWo"], dbqkv=o["dbqkv"], dX_handoff=o["dXah"])


@pytest.mark.parametrize("streams", [1])
def test_captured_layer_step_replays_the_eager_bits(streams):
    w = LAYER
    print(f"[case] graph capture {w.key} streams={streams}", flush=True)
    inp = synth.make_inputs(w)
    d = {k: v.to("cuda").contiguous() for k, v in inp.items()}
    with T.plan_for(w, n_streams=streams, handoff_rows=True) as p:
        o = _outputs(p.info)
        _step(p, d, o)  # eager, also makes the plan's workspaces and events
        torch.cuda.synchronize()
        ref = {k: v.clone() for k, v in o.items()}
        for v in o.values():
            v.fill_(float("nan"))
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s), torch.cuda.graph(g, stream=s):
            _step(p, d, o)
        torch.cuda.synchronize()
        for rep in range(3):
            for v in o.values():
                v.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for k in o:
                assert torch.equal(o[k], ref[k]), (rep, k)
            # eager work of the program between replays
            x = torch.randn(256, 256, device="cuda")
            (x @ x).sum().item()
        del g
        torch.cuda.synchronize()
    for k in ("Zah", "Zh", "dXh", "dXah"):
        assert torch.equal(ref[k], ref[k[:-1]]), k


@pytest.mark.parametrize("kw", [dict(n_streams=2), dict(pipeline=True)], ids=["two_streams", "pipelined"])
def test_capture_of_other_plans_is_refused_before_any_work(kw):
    """A plan with two worker streams, or a pipelined one, called on a capturing stream: the call
    returns TPSLICE_ERR_UNSUPPORTED before it queues anything (the captured graph holds only the
    caller's own work)."""
    w = LAYER
    print(f"[case] graph capture refused {kw}", flush=True)
    inp = synth.make_inputs(w)
    d = {k: v.to("cuda").contiguous() for k, v in inp.items()}
    with T.plan_for(w, handoff_rows=True, **kw) as p:
        o = _outputs(p.info)
        p.mlp_fwd(d["X_mlp"], d["W1"], d["b1"], d["W2"], o["Z"], o["U"], o["Zh"])  # eager: accepted
        p.handoff_wait()
        torch.cuda.synchronize()
        x = torch.zeros(16, device="cuda")
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s), torch.cuda.graph(g, stream=s):
            x.add_(1.0)
            with pytest.raises(T.TpsliceError) as e:
                p.mlp_fwd(d["X_mlp"], d["W1"], d["b1"], d["W2"], o["Z"], o["U"], o["Zh"])
        assert e.value.code == T.ERR_UNSUPPORTED
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(x, torch.ones(16, device="cuda"))
        del g
