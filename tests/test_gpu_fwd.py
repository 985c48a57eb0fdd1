"""GPU parity of the chunked forward pass and of the fp32 recurrent reference
against the CPU fp64 oracle, through the C ABI (marked gpu).

Tolerances (tests/golden/page_constants.json): max-relative error <= 3e-4 for
fp32 io (true fp32 compute), relative RMS <= 8e-3 for bf16 operands with an
fp32 state (the 0.008 output threshold of the fla issue #1550 page), each on
the output and on the final state separately.
"""
import json
import os

import numpy as np
import pytest
import torch

import gated_deltanet_chunked_gdn_amd as gdn
from gated_deltanet_chunked_gdn_amd.workloads import WORKLOADS, Workload, generate
from _helpers import max_rel, oracle_fwd, rel_rms, report, to_device, to_np, worst_head_rel_rms

pytestmark = pytest.mark.gpu

_C = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))
TOL_BF16 = _C["tolerance_rel_rms_bf16"]["value"]
TOL_FP32 = _C["tolerance_max_rel_fp32"]["value"]


def run_chunk(d, **kw):
    t = to_device(d)
    o, Sf = gdn.chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=t.get("S0"),
                          cu_seqlens=d["cu_seqlens"], scale=d["scale"], **kw)
    torch.cuda.synchronize()
    return to_np(o), to_np(Sf)


def check_against_oracle(name, d, o, Sf):
    o_ref, S_ref = oracle_fwd(d)
    if d["io"] == "fp32":
        eo, es = max_rel(o, o_ref), max_rel(Sf, S_ref)
        report(name, o_max_rel=eo, S_max_rel=es)
        assert eo <= TOL_FP32 and es <= TOL_FP32
    else:
        eo, es = rel_rms(o, o_ref), rel_rms(Sf, S_ref)
        # the worst (sequence, head): a whole-tensor value can hide one bad head
        ho = worst_head_rel_rms(o, o_ref, cu_seqlens=d["cu_seqlens"])
        hs = worst_head_rel_rms(Sf, S_ref, token_major=False)
        report(name, o_rel_rms=eo, S_rel_rms=es, o_worst_head=ho, S_worst_head=hs)
        assert eo <= TOL_BF16 and es <= TOL_BF16
        assert ho <= TOL_BF16 and hs <= TOL_BF16
    return o_ref, S_ref


@pytest.mark.parametrize("name", ["tiny_fp32", "train_bf16", "packed_bf16", "fwdbwd_bf16"])
def test_chunk_fwd_named_workloads(name):
    d = generate(WORKLOADS[name])
    o, Sf = run_chunk(d)
    check_against_oracle(name, d, o, Sf)


def test_chunk_fwd_long_serial_per_window():
    """Slow decay over 65536 tokens, serial over chunks; rel-L2 per 8K window
    (the windows of the cuLA issue #126 page, "Minimal public reproduction")."""
    d = generate(WORKLOADS["long_bf16"])
    o, Sf = run_chunk(d)
    o_ref, S_ref = check_against_oracle("long_bf16 serial", d, o, Sf)
    for w in range(8):
        sl = slice(8192 * w, 8192 * (w + 1))
        e = rel_rms(o[:, sl], o_ref[:, sl])
        report(f"  window {w}", rel_l2=e)
        assert e <= TOL_BF16


CASES = [
    # (B, T, H, Dk, Dv, io, cu_seqlens, s0, scale, gate)
    (1, 1, 1, 64, 64, "fp32", None, 0.5, 1.0, "softplus01"),
    (2, 63, 2, 64, 32, "fp32", None, 0.5, 0.125, "gdn"),
    (1, 100, 3, 64, 64, "fp32", (0, 0, 37, 100), 0.3, 0.7, "bounded5"),
    (1, 65, 1, 128, 16, "bf16", None, None, 1.0, "gdn"),
    (3, 100, 2, 128, 48, "bf16", None, 0.1, 128 ** -0.5, "gdn"),
    (1, 4097, 2, 128, 128, "bf16", None, 0.1, 1.0, "gdn"),
    (1, 4197, 2, 128, 128, "bf16", (0, 100, 4197), 0.1, 1.0, "bounded5"),
    (1, 300, 2, 64, 256, "bf16", (0, 64, 64, 129, 300), 0.2, 1.0, "softplus01"),
    (2, 640, 4, 64, 128, "bf16", None, None, 1.0, "const"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}k{c[3]}v{c[4]}{c[5]}")
def test_chunk_fwd_shapes_and_edges(case):
    B, T, H, Dk, Dv, io, cu, s0, scale, gate = case
    w = Workload("case", B, T, H, Dk, Dv, io=io, qk="norm_both", gate=gate, cu_seqlens=cu,
                 s0_std=s0, scale=scale, seed=T + Dv)
    d = generate(w)
    o, Sf = run_chunk(d)
    check_against_oracle(f"case {case}", d, o, Sf)


def test_beta_near_two_and_strong_decay():
    w = Workload("b2", 2, 200, 2, 128, 64, io="bf16", qk="norm_both", gate="bounded5", s0_std=0.1)
    d = generate(w)
    d["beta"] = (1.99 * d["beta"]).astype(np.float32)
    o, Sf = run_chunk(d)
    check_against_oracle("beta~2", d, o, Sf)


def test_empty_sequences_and_zero_tokens():
    w = Workload("empty", 1, 0, 2, 64, 32, io="bf16", cu_seqlens=(0, 0, 0), s0_std=0.1)
    d = generate(w)
    o, Sf = run_chunk(d)
    assert o.size == 0
    np.testing.assert_array_equal(Sf, d["S0"])


def test_packed_equals_dense_and_resume_and_determinism():
    """Bitwise invariants: packed == each sequence alone; resuming at a chunk
    boundary == one call; two runs give the same bits."""
    w = Workload("inv", 1, 384, 3, 128, 64, io="bf16", qk="norm_both", gate="gdn",
                 cu_seqlens=(0, 128, 384), s0_std=0.1, seed=5)
    d = generate(w)
    o, Sf = run_chunk(d)
    o2, Sf2 = run_chunk(d)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(Sf, Sf2)
    t = to_device(d)
    for n, (a, b) in enumerate([(0, 128), (128, 384)]):
        on, Sn = gdn.chunk_fwd(*(t[x][:, a:b].contiguous() for x in ("q", "k", "v", "g", "beta")),
                               S0=t["S0"][n:n + 1].contiguous())
        np.testing.assert_array_equal(to_np(on), o[:, a:b])
        np.testing.assert_array_equal(to_np(Sn), Sf[n:n + 1])
    # resume the second sequence after 64 tokens
    a, m, b = 128, 192, 384
    oa, Sa = gdn.chunk_fwd(*(t[x][:, a:m].contiguous() for x in ("q", "k", "v", "g", "beta")),
                           S0=t["S0"][1:2].contiguous())
    ob, Sb = gdn.chunk_fwd(*(t[x][:, m:b].contiguous() for x in ("q", "k", "v", "g", "beta")),
                           S0=Sa)
    np.testing.assert_array_equal(np.concatenate([to_np(oa), to_np(ob)], axis=1), o[:, a:b])
    np.testing.assert_array_equal(to_np(Sb), Sf[1:2])


def test_nan_stays_in_its_head():
    w = Workload("nan", 2, 130, 3, 64, 64, io="bf16", qk="norm_both", gate="gdn")
    d = generate(w)
    d["v"][1, 70, 2, 5] = np.nan
    o, Sf = run_chunk(d)
    bad = np.zeros(o.shape, bool)
    bad[1, :, 2] = True
    assert np.all(np.isfinite(o[~bad]))
    assert np.all(np.isfinite(Sf[[0, 0, 0, 1, 1], [0, 1, 2, 0, 1]]))


@pytest.mark.parametrize("name", ["tiny_fp32", "train_bf16", "packed_bf16"])
def test_recurrent_ref_forward(name):
    d = generate(WORKLOADS[name])
    t = to_device(d)
    out = gdn.recurrent_ref(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=t.get("S0"),
                            cu_seqlens=d["cu_seqlens"], scale=d["scale"])
    torch.cuda.synchronize()
    o, Sf = to_np(out["o"]), to_np(out["S_final"])
    o_ref, S_ref = oracle_fwd(d)
    eo, es = max_rel(o, o_ref), max_rel(Sf, S_ref)
    report(f"recurrent {name}", o_max_rel=eo, S_max_rel=es, o_rel_rms=rel_rms(o, o_ref))
    assert es <= TOL_FP32  # fp32 state throughout
    if d["io"] == "fp32":
        assert eo <= TOL_FP32
    else:  # only the final bf16 rounding of o remains
        assert rel_rms(o, o_ref) <= 3e-3
