"""GPU parity of the chunked backward pass (gdn_chunk_bwd) against the oracle's
fp64 reverse mode, and against the fp32 recurrent reference at full length
(marked gpu).

Gradients of L = <o, dO> + <S_final, dS_final> with respect to q, k, v, g,
beta and S0.  Tolerances as for the forward (tests/golden/page_constants.json):
max-relative <= 3e-4 for fp32 io, relative RMS <= 8e-3 for bf16 io, each
gradient separately.
"""
import json
import os

import numpy as np
import pytest
import torch

import gated_deltanet_chunked_gdn_amd as gdn
import oracle
from gated_deltanet_chunked_gdn_amd.workloads import WORKLOADS, Workload, generate
from _helpers import max_rel, rel_rms, report, to_device, to_np, truncate
from oracle.compare import rel_rms_per_head

pytestmark = pytest.mark.gpu

_C = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))
TOL_BF16 = _C["tolerance_rel_rms_bf16"]["value"]
TOL_FP32 = _C["tolerance_max_rel_fp32"]["value"]
GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


def chunk_bwd(d, dS_final=None):
    t = to_device(d)
    dSf = None if dS_final is None else torch.from_numpy(dS_final).cuda()
    out = gdn.chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dO"], S0=t.get("S0"),
                        dS_final=dSf, cu_seqlens=d["cu_seqlens"], scale=d["scale"])
    torch.cuda.synchronize()
    return {k: to_np(v) for k, v in out.items()}


def oracle_bwd(d, dS_final=None):
    return oracle.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["dO"], cu_seqlens=d["cu_seqlens"],
                      S0=d["S0"], dS_final=dS_final, scale=d["scale"])


def head_sensitivity(d, dS_final=None, ref=None):
    """Per-(sequence, head) rel-RMS by which the oracle's gradients move when the
    bf16 inputs q, k, v, dO are perturbed by independent relative noise of up to
    one bf16 unit roundoff (2^-9): how ill-conditioned each head's gradients are
    under the rounding the fla issue #1550 page blames ("Intermediate rounding
    diagnosis").  A head whose gradient nearly cancels (strong decay, a small
    dg or dbeta) moves by more than the tensor as a whole."""
    rng = np.random.default_rng(2024)
    p = dict(d)
    for key in ("q", "k", "v", "dO"):
        x = d[key].astype(np.float64)
        p[key] = x * (1.0 + 2.0 ** -9 * rng.uniform(-1.0, 1.0, size=x.shape))
    ref = oracle_bwd(d, dS_final) if ref is None else ref
    pert = oracle_bwd(p, dS_final)
    like = {"dq": "q", "dk": "k", "dv": "v", "dg": "g", "dbeta": "beta"}
    out = {}
    for g in GRADS:
        shape = d[like[g]].shape if g in like else ref[g].shape
        out[g] = rel_rms_per_head(pert[g].reshape(shape), ref[g].reshape(shape), cu_seqlens=d["cu_seqlens"],
                                  token_major=g != "dS0")
    return out


def check(name, d, out, ref, dS_final=None):
    sens = head_sensitivity(d, dS_final, ref) if d["io"] != "fp32" else None
    for g in GRADS:
        r = ref[g].reshape(out[g].shape)
        if d["io"] == "fp32":
            e = max_rel(out[g], r)
            report(f"{name} {g}", max_rel=e)
            assert e <= TOL_FP32, g
        else:
            e = rel_rms(out[g], r)
            # every (sequence, head) separately, too: a whole-tensor value can hide
            # one bad head.  A head is held to the tensor bound, or to 4x what
            # bf16-sized noise on the inputs alone does to that head when its
            # gradient is that ill-conditioned.
            per = rel_rms_per_head(out[g], r, cu_seqlens=d["cu_seqlens"], token_major=g != "dS0")
            bound = np.maximum(TOL_BF16, 4.0 * sens[g].reshape(per.shape))
            worst = int(np.argmax(per / bound)) if per.size else 0
            report(f"{name} {g}", rel_rms=e, worst_head=float(per.max()) if per.size else 0.0,
                   worst_head_over_bound=float((per / bound).flat[worst]) if per.size else 0.0)
            assert e <= TOL_BF16, g
            assert np.all(per <= bound), (g, per, bound)


def test_chunk_bwd_training_slice_vs_oracle():
    """The value-expansion-2 training shape (B=32, T=1024, H=16, d_k=64, d_v=128),
    first 256 tokens, S0 = 0 passed explicitly."""
    d = truncate(generate(WORKLOADS["fwdbwd_bf16"]), 256)
    check("fwdbwd_bf16[:256]", d, chunk_bwd(d), oracle_bwd(d))


def test_chunk_bwd_training_full_vs_recurrent():
    """Full length (T=1024): the chunked backward against the fp32 recurrent
    reverse mode on the GPU (the oracle covers the 256-token slice)."""
    d = generate(WORKLOADS["fwdbwd_bf16"])
    out = chunk_bwd(d)
    t = to_device(d)
    ref = gdn.recurrent_ref(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=t["S0"], scale=d["scale"],
                            dO=t["dO"])
    torch.cuda.synchronize()
    for g in GRADS:
        e = rel_rms(out[g], to_np(ref[g]))
        report(f"fwdbwd_bf16 full vs recurrent {g}", rel_rms=e)
        assert e <= TOL_BF16, g


CASES = [
    # (B, T, H, Dk, Dv, io, cu_seqlens, s0, scale, gate, with dS_final)
    (1, 1, 1, 64, 64, "fp32", None, 0.5, 1.0, "softplus01", True),
    (2, 63, 2, 64, 32, "fp32", None, None, 0.25, "gdn", False),
    (1, 200, 3, 64, 64, "fp32", (0, 0, 37, 200), 0.3, 0.7, "bounded5", True),
    (2, 130, 2, 64, 16, "fp32", None, 0.2, 1.0, "gdn", True),
    (1, 300, 2, 128, 64, "fp32", (0, 70, 70, 300), 0.2, 0.5, "gdn", True),
    (1, 65, 1, 128, 16, "bf16", None, None, 1.0, "gdn", False),
    (3, 100, 2, 128, 48, "bf16", None, 0.1, 128 ** -0.5, "gdn", True),
    (1, 300, 2, 64, 256, "bf16", (0, 64, 64, 129, 300), 0.2, 1.0, "softplus01", True),
    (2, 640, 4, 128, 128, "bf16", None, None, 1.0, "const", False),
    (1, 777, 2, 128, 80, "bf16", (0, 500, 777), 0.1, 1.0, "bounded5", True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}k{c[3]}v{c[4]}{c[5]}")
def test_chunk_bwd_shapes_and_edges(case):
    B, T, H, Dk, Dv, io, cu, s0, scale, gate, with_dsf = case
    w = Workload("bwd", B, T, H, Dk, Dv, io=io, qk="norm_both", gate=gate, cu_seqlens=cu,
                 s0_std=s0, scale=scale, with_dO=True, seed=T + Dv + 7)
    d = generate(w)
    dSf = None
    if with_dsf:
        dSf = np.random.default_rng(T).standard_normal((w.num_seqs, H, Dk, Dv)).astype(np.float32)
    check(f"bwd {case}", d, chunk_bwd(d, dSf), oracle_bwd(d, dSf), dSf)


def test_chunk_bwd_beta_near_two_strong_decay():
    w = Workload("bwd", 2, 257, 2, 64, 64, io="bf16", qk="norm_both", gate="bounded5",
                 s0_std=0.2, with_dO=True, seed=21)
    d = generate(w)
    d["beta"] = np.full_like(d["beta"], 1.9)
    check("bwd beta=1.9", d, chunk_bwd(d), oracle_bwd(d))


def test_chunk_bwd_deterministic_and_packed_equals_dense():
    w = Workload("bwd", 2, 300, 2, 128, 64, io="bf16", qk="norm_both", gate="gdn", s0_std=0.1,
                 with_dO=True, seed=5)
    d = generate(w)
    a, b = chunk_bwd(d), chunk_bwd(d)
    for g in GRADS:
        assert np.array_equal(a[g], b[g]), g
    # the same two sequences packed into one row
    p = dict(d)
    for key in ("q", "k", "v", "g", "beta", "dO"):
        p[key] = np.ascontiguousarray(d[key].reshape((1, 600) + d[key].shape[2:]))
    p["cu_seqlens"] = np.array([0, 300, 600], dtype=np.int32)
    c = chunk_bwd(p)
    for g in ("dq", "dk", "dv", "dg", "dbeta"):
        assert np.array_equal(c[g].reshape(a[g].shape), a[g]), g
    assert np.array_equal(c["dS0"], a["dS0"])
