"""gdn_chunk_fwd_noalloc against gdn_chunk_fwd, through the C ABI (marked gpu).

The no-allocation entry point runs gdn_chunk_fwd's kernels with the library's
fixed device workspace.  On the same inputs its outputs must equal those of
gdn_chunk_fwd with a caller-provided workspace bit for bit; two calls in a row
(the second smaller, so it runs over what the first left in the shared array)
are both checked, the smaller one also against the fp64 oracle.  A problem too
large for the array is refused before any launch, and a captured call replays
like the eager one.
"""
import pytest
import torch

import gated_deltanet_chunked_gdn_amd as gdn
from gated_deltanet_chunked_gdn_amd import _native as nat
from gated_deltanet_chunked_gdn_amd.ops import SeqLens
from gated_deltanet_chunked_gdn_amd.workloads import WORKLOADS, Workload, generate
from _helpers import oracle_fwd, rel_rms, report, to_device, to_np

pytestmark = pytest.mark.gpu


def _both(d, num_segments=1):
    t = to_device(d)
    seqs = SeqLens(d["cu_seqlens"], t["q"].device) if d["cu_seqlens"] is not None else None
    o_ref, S_ref = gdn.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=t.get("S0"), cu_seqlens=seqs,
                                 scale=d["scale"], num_segments=num_segments)
    o = torch.full_like(o_ref, float("nan"))
    Sf = torch.full_like(S_ref, float("nan"))
    gdn.chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"], out=o, final_state_out=Sf,
                          S0=t.get("S0"), cu_seqlens=seqs, scale=d["scale"], num_segments=num_segments)
    torch.cuda.synchronize()
    return (o, Sf), (o_ref, S_ref), t


def _same_bits(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def test_noalloc_matches_chunk_fwd_two_calls_second_smaller():
    print("noalloc call 1: train_bf16 B4 T4096 H8 d128", flush=True)
    d1 = generate(WORKLOADS["train_bf16"])
    (o1, S1), (o1r, S1r), _ = _both(d1)
    assert _same_bits(o1, o1r) and _same_bits(S1, S1r)

    print("noalloc call 2: packed T300 cu [0,100,300] H2 d128, S0, scale 0.5", flush=True)
    w2 = Workload("noalloc_small", 1, 300, 2, 128, 128, io="bf16", qk="norm_both", gate="gdn",
                  cu_seqlens=(0, 100, 300), s0_std=0.1, scale=0.5, seed=21)
    d2 = generate(w2)
    (o2, S2), (o2r, S2r), _ = _both(d2)
    assert _same_bits(o2, o2r) and _same_bits(S2, S2r)
    oo, so = oracle_fwd(d2)
    eo, es = rel_rms(to_np(o2), oo), rel_rms(to_np(S2), so)
    report("noalloc small vs oracle", o_rel_rms=eo, S_rel_rms=es)
    assert eo <= 8e-3 and es <= 8e-3


def test_noalloc_segment_split_and_fp32():
    print("noalloc: long slice T8192 H1 d128, G=4", flush=True)
    d = generate(WORKLOADS["long_bf16"].with_(T=8192))
    (o, S), (o_r, S_r), _ = _both(d, num_segments=4)
    assert _same_bits(o, o_r) and _same_bits(S, S_r)
    print("noalloc: tiny_fp32", flush=True)
    d = generate(WORKLOADS["tiny_fp32"])
    (o, S), (o_r, S_r), _ = _both(d)
    assert _same_bits(o, o_r) and _same_bits(S, S_r)


def test_noalloc_refuses_oversize_problem_before_launch():
    print("noalloc: oversize problem refused", flush=True)
    dev = torch.device("cuda")
    B, T, H, Dk, Dv = 32, 1024, 16, 64, 128     # needs ~126 MiB of workspace
    q = torch.zeros(B, T, H, Dk, dtype=torch.bfloat16, device=dev)
    v = torch.zeros(B, T, H, Dv, dtype=torch.bfloat16, device=dev)
    g = torch.zeros(B, T, H, dtype=torch.float32, device=dev)
    out = torch.full_like(v, 7.0)
    with pytest.raises(nat.GdnError) as e:
        gdn.chunk_fwd_noalloc(q, q.clone(), v, g, g.clone(), out=out)
    assert e.value.status == nat.GDN_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


def test_noalloc_graph_replay_matches_eager():
    print("noalloc: captured call replayed", flush=True)
    w = Workload("noalloc_graph", 2, 640, 3, 128, 128, io="bf16", qk="norm_both", gate="gdn", seed=23)
    d = generate(w)
    t = to_device(d)
    o_eager = torch.empty_like(t["v"])
    S_eager = torch.empty(2, 3, 128, 128, dtype=torch.float32, device=t["q"].device)
    gdn.chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"], out=o_eager, final_state_out=S_eager)
    torch.cuda.synchronize()
    o = torch.empty_like(o_eager)
    S = torch.empty_like(S_eager)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdn.chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"], out=o, final_state_out=S)
    torch.cuda.synchronize()
    for r in range(3):
        o.fill_(float("nan"))
        S.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert _same_bits(o, o_eager) and _same_bits(S, S_eager), f"replay {r}"
        # eager work on the shared array between replays
        gdn.chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"], out=torch.empty_like(o))
        torch.cuda.synchronize()
