"""HIP-graph capture and replay of the chunked forward and backward passes and
of the per-key-channel-decay forward, backward and retained-state training step
(marked gpu).

The library allocates nothing and issues no memset, so a call can be captured
into a graph.  Each test captures one call, then replays the graph several times
with new input values copied in between (eager work and synchronisations between
the replays), and checks every replay bit-for-bit against an eager call on the
same inputs: the kernels are deterministic.  Reproducibility questions of the
pages: "Research Sprint Day 1", "Open questions", and the fla issue #1550 page,
"Proposed scope" (graph-captured training steps).
"""
import numpy as np
import pytest
import torch

import gated_deltanet_chunked_gdn_amd as gdn
from gated_deltanet_chunked_gdn_amd.workloads import Workload, generate
from _helpers import to_device

pytestmark = pytest.mark.gpu

W = Workload("graph", 2, 300, 3, 128, 64, io="bf16", qk="norm_both", gate="gdn", s0_std=0.1,
             with_dO=True, scale=0.5, seed=31)


def _inputs(seed):
    d = generate(Workload(**{**W.__dict__, "seed": seed}))
    return d, to_device(d)


def _copy_into(dst, src):
    for key in dst:
        dst[key].copy_(src[key])


def test_forward_graph_replays_match_eager():
    d, t = _inputs(31)
    dev = t["q"].device
    o = torch.empty_like(t["v"])
    Sf = torch.empty((W.B, W.H, W.Dk, W.Dv), dtype=torch.float32, device=dev)
    ws = gdn.forward_workspace(t["q"], t["v"])

    def call():
        gdn.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=t["S0"], scale=W.scale,
                      out=o, final_state_out=Sf, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep, seed in enumerate((32, 33, 34)):
        _, fresh = _inputs(seed)
        _copy_into(t, fresh)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_graph, S_graph = o.clone(), Sf.clone()
        o_eager, S_eager = gdn.chunk_fwd(fresh["q"], fresh["k"], fresh["v"], fresh["g"], fresh["beta"],
                                         S0=fresh["S0"], scale=W.scale)
        torch.cuda.synchronize()
        assert torch.equal(o_graph, o_eager), f"replay {rep}: output differs from the eager call"
        assert torch.equal(S_graph, S_eager), f"replay {rep}: final state differs from the eager call"
        assert np.isfinite(o_graph.float().cpu().numpy()).all()


def test_backward_graph_replays_match_eager():
    d, t = _inputs(41)
    result = {}

    def call():
        result.update(gdn.chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dO"], S0=t["S0"],
                                    scale=W.scale))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep, seed in enumerate((42, 43)):
        _, fresh = _inputs(seed)
        _copy_into(t, fresh)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in result.items()}
        ref = gdn.chunk_bwd(fresh["q"], fresh["k"], fresh["v"], fresh["g"], fresh["beta"], fresh["dO"],
                            S0=fresh["S0"], scale=W.scale)
        torch.cuda.synchronize()
        for name in ("dq", "dk", "dv", "dg", "dbeta", "dS0"):
            assert torch.equal(got[name], ref[name]), f"replay {rep}: {name} differs from the eager call"


def test_kda_forward_graph_replays_match_eager():
    # the per-key-channel-decay forward, captured once and replayed on new inputs
    wk = Workload("graph_kda", 2, 300, 3, 128, 64, io="bf16", qk="norm_both", gate="gdn_channel", s0_std=0.1,
                  scale=0.5, seed=51)

    def inputs(seed):
        return to_device(generate(Workload(**{**wk.__dict__, "seed": seed})))

    t = inputs(51)
    dev = t["q"].device
    o = torch.empty_like(t["v"])
    Sf = torch.empty((wk.B, wk.H, wk.Dk, wk.Dv), dtype=torch.float32, device=dev)
    from gated_deltanet_chunked_gdn_amd import _native as nat
    ws = torch.empty(nat.workspace_size(gdn.make_problem(t["q"], t["v"], None, 1.0, 1), nat.GDN_PASS_KDA_FWD),
                     dtype=torch.uint8, device=dev)

    def call():
        gdn.kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=t["S0"], scale=wk.scale, out=o,
                          final_state_out=Sf, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep, seed in enumerate((52, 53, 54)):
        fresh = inputs(seed)
        _copy_into(t, fresh)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_graph, S_graph = o.clone(), Sf.clone()
        o_eager, S_eager = gdn.kda_chunk_fwd(fresh["q"], fresh["k"], fresh["v"], fresh["g"], fresh["beta"],
                                             S0=fresh["S0"], scale=wk.scale)
        torch.cuda.synchronize()
        assert torch.equal(o_graph, o_eager), f"replay {rep}: output differs from the eager call"
        assert torch.equal(S_graph, S_eager), f"replay {rep}: final state differs from the eager call"


def test_kda_training_step_graph_replays_match_eager():
    # a per-key-channel-decay training step with retained states (forward with
    # save, then the backward from the saved buffer) captured as one graph, and
    # the recomputing backward captured alone: every replay on new inputs equals
    # the eager calls bit for bit
    wk = Workload("graph_kda_bwd", 2, 300, 3, 128, 64, io="bf16", qk="norm_both", gate="gdn_channel",
                  s0_std=0.1, with_dO=True, scale=0.5, seed=61)

    def inputs(seed):
        return to_device(generate(Workload(**{**wk.__dict__, "seed": seed})))

    t = inputs(61)
    saved = gdn.kda_saved_buffer(t["q"], t["v"])
    step, recompute = {}, {}

    def call_step():
        o, Sf, _ = gdn.kda_chunk_fwd_save(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=t["S0"], scale=wk.scale,
                                          saved=saved)
        step.update(gdn.kda_chunk_bwd_saved(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dO"], saved,
                                            scale=wk.scale))
        step["o"], step["Sf"] = o, Sf

    def call_bwd():
        recompute.update(gdn.kda_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dO"], S0=t["S0"],
                                           scale=wk.scale))

    graphs = []
    for call in (call_step, call_bwd):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call()
        torch.cuda.synchronize()
        graphs.append(graph)
    for rep, seed in enumerate((62, 63)):
        fresh = inputs(seed)
        _copy_into(t, fresh)
        torch.cuda.synchronize()
        for graph in graphs:
            graph.replay()
        torch.cuda.synchronize()
        got_step = {k: v.clone() for k, v in step.items()}
        got_bwd = {k: v.clone() for k, v in recompute.items()}
        o_ref, Sf_ref = gdn.kda_chunk_fwd(fresh["q"], fresh["k"], fresh["v"], fresh["g"], fresh["beta"],
                                          S0=fresh["S0"], scale=wk.scale)
        ref = gdn.kda_chunk_bwd(fresh["q"], fresh["k"], fresh["v"], fresh["g"], fresh["beta"], fresh["dO"],
                                S0=fresh["S0"], scale=wk.scale)
        torch.cuda.synchronize()
        assert torch.equal(got_step["o"], o_ref) and torch.equal(got_step["Sf"], Sf_ref), f"replay {rep}: forward"
        for name in ("dq", "dk", "dv", "dg", "dbeta", "dS0"):
            assert torch.equal(got_step[name], ref[name]), f"replay {rep}: retained {name} differs from eager"
            assert torch.equal(got_bwd[name], ref[name]), f"replay {rep}: recomputing {name} differs from eager"
