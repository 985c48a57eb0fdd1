"""GPU checks of training with retained states (gdn_chunk_fwd_save +
gdn_chunk_bwd_saved), marked gpu.

The forward that keeps the backward's records runs the same arithmetic as
gdn_chunk_fwd, and the backward from them the same as the reverse passes of
gdn_chunk_bwd, whose state pass recomputes exactly the states the forward kept.
So o, S_final and every gradient must be bit-identical to the recomputing path
(itself checked against the fp64 oracle in test_gpu_chunk_bwd.py and
test_gpu_fwd.py); one case is also compared with the oracle directly.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_chunked_gdn_amd as gdn
import oracle
from gated_deltanet_chunked_gdn_amd.workloads import WORKLOADS, Workload, generate
from _helpers import max_rel, rel_rms, report, to_device, to_np, truncate

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dS0")

CASES = [
    # (B, T, H, Dk, Dv, io, cu_seqlens, s0, gate, with dS_final)
    (1, 1, 1, 64, 64, "fp32", None, 0.5, "softplus01", True),
    (2, 130, 2, 64, 16, "fp32", None, 0.2, "gdn", True),
    (1, 200, 2, 128, 32, "fp32", (0, 1, 65, 200), 0.2, "gdn", True),
    (1, 65, 1, 128, 16, "bf16", None, None, "gdn", False),
    (3, 100, 2, 128, 48, "bf16", None, 0.1, "gdn", True),
    (1, 300, 2, 64, 256, "bf16", (0, 64, 64, 129, 300), 0.2, "softplus01", True),
    (2, 640, 4, 128, 128, "bf16", None, None, "const", False),
    (1, 777, 2, 128, 80, "bf16", (0, 500, 777), 0.1, "bounded5", True),
]


def both_paths(d, dSf=None, saved=None):
    t = to_device(d)
    dS = None if dSf is None else torch.from_numpy(dSf).cuda()
    kw = dict(cu_seqlens=d["cu_seqlens"], scale=d["scale"])
    o1, S1 = gdn.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=t.get("S0"), **kw)
    g1 = gdn.chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dO"], S0=t.get("S0"), dS_final=dS, **kw)
    o2, S2, sv = gdn.chunk_fwd_save(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=t.get("S0"), saved=saved, **kw)
    g2 = gdn.chunk_bwd_saved(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dO"], sv, dS_final=dS, **kw)
    torch.cuda.synchronize()
    return (to_np(o1), to_np(S1), {k: to_np(v) for k, v in g1.items()},
            to_np(o2), to_np(S2), {k: to_np(v) for k, v in g2.items()}, sv)


def assert_identical(name, res):
    o1, S1, g1, o2, S2, g2, _ = res
    assert np.array_equal(o1, o2), f"{name} o"
    assert np.array_equal(S1, S2), f"{name} S_final"
    for g in GRADS:
        assert np.array_equal(g1[g], g2[g]), f"{name} {g}"


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}k{c[3]}v{c[4]}{c[5]}")
def test_saved_path_bit_identical(case):
    B, T, H, Dk, Dv, io, cu, s0, gate, with_dsf = case
    w = Workload("saved", B, T, H, Dk, Dv, io=io, qk="norm_both", gate=gate, cu_seqlens=cu,
                 s0_std=s0, with_dO=True, seed=T + Dk + 3)
    d = generate(w)
    dSf = None
    if with_dsf:
        dSf = np.random.default_rng(T + 1).standard_normal((w.num_seqs, H, Dk, Dv)).astype(np.float32)
    res = both_paths(d, dSf)
    assert_identical(f"saved {case}", res)


def test_saved_training_shape_and_buffer_reuse():
    """fwdbwd_bf16 (B=32, T=1024, H=16, d_k=64, d_v=128): bit-identical to the
    recomputing path; then a second step with other inputs through the same
    buffer (whatever the first step left in it is overwritten)."""
    d = generate(WORKLOADS["fwdbwd_bf16"])
    res = both_paths(d)
    assert_identical("fwdbwd_bf16", res)
    sv = res[6]
    w2 = Workload("fwdbwd2", 32, 1024, 16, 64, 128, io="bf16", qk="norm_both", gate="gdn",
                  s0_std=0.1, with_dO=True, seed=99)
    res2 = both_paths(generate(w2), saved=sv)
    assert_identical("fwdbwd_bf16 second step", res2)
    assert res2[6].data_ptr() == sv.data_ptr()


def test_saved_vs_oracle():
    d = truncate(generate(WORKLOADS["fwdbwd_bf16"]), 256)
    _, _, _, o2, S2, g2, _ = both_paths(d)
    ref = oracle.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["dO"], cu_seqlens=d["cu_seqlens"],
                     S0=d["S0"], scale=d["scale"])
    o_ref, _ = oracle.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                          S0=d["S0"], scale=d["scale"])
    e = rel_rms(o2, o_ref.reshape(o2.shape))
    report("saved fwdbwd_bf16[:256] o", rel_rms=e)
    assert e <= 8e-3
    for g in GRADS:
        e = rel_rms(g2[g], ref[g].reshape(g2[g].shape))
        report(f"saved fwdbwd_bf16[:256] {g}", rel_rms=e)
        assert e <= 8e-3, g
