"""GPU parity of the fused input prologue (gdn_prologue) against the oracle's
float64 prologue, through the C ABI (marked gpu).

Bounds: the normalised q and k are one rounding of the fp32 result to the io
dtype, so each element is within 2^-8 of the float64 value relative to it for
bf16 (2^-9 for the rounding, the rest for fp32 arithmetic) and within 4e-7 for
fp32; g and beta are fp32 expressions with exponentials, within 1e-5 relative.
The end-to-end check feeds the prologue's outputs to the chunked forward and
compares with the oracle run on the same (prologue-made) inputs.
"""
import json
import os

import numpy as np
import pytest
import torch

import gated_deltanet_chunked_gdn_amd as gdn
import oracle
from gated_deltanet_chunked_gdn_amd.workloads import round_bf16
from _helpers import rel_rms, report

pytestmark = pytest.mark.gpu

_C = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))
TOL_BF16 = _C["tolerance_rel_rms_bf16"]["value"]


def _raw(B, T, H, Dk, io, seed):
    rng = np.random.default_rng(seed)
    f = np.float32
    q = rng.standard_normal((B, T, H, Dk), dtype=f) * f(3.0)
    k = rng.standard_normal((B, T, H, Dk), dtype=f) * f(0.2)
    if io == "bf16":
        q, k = round_bf16(q), round_bf16(k)
    a = rng.standard_normal((B, T, H), dtype=f)
    b = rng.standard_normal((B, T, H), dtype=f) * f(2.0)
    A_log = rng.uniform(0.0, 1.5, size=(H,)).astype(f)
    dt = (f(0.5) * rng.standard_normal(H, dtype=f)).astype(f)
    return q, k, a, b, A_log, dt


def _dev(x, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype)


@pytest.mark.parametrize("B,T,H,Dk,io,gate,neg", [
    (1, 1, 1, 64, "bf16", "gdn", False),
    (2, 77, 3, 128, "bf16", "gdn", True),
    (1, 300, 5, 64, "bf16", "bounded5", False),
    (3, 65, 2, 128, "fp32", "gdn", False),
    (1, 129, 4, 64, "fp32", "bounded5", True),
    (4, 4096, 8, 128, "bf16", "gdn", False),
])
def test_prologue_matches_oracle(B, T, H, Dk, io, gate, neg):
    q, k, a, b, A_log, dt = _raw(B, T, H, Dk, io, seed=B * 1000 + T)
    iot = torch.bfloat16 if io == "bf16" else torch.float32
    qo, ko, g, beta = gdn.prologue(_dev(q, iot), _dev(k, iot), _dev(a), _dev(b), _dev(A_log), _dev(dt),
                                   gate=gate, allow_neg_eigval=neg)
    torch.cuda.synchronize()
    rq, rk, rg, rb = oracle.prologue(q, k, a, b, A_log, dt, gate=gate, allow_neg_eigval=neg)
    rel = 2.0 ** -8 if io == "bf16" else 4e-7
    for name, got, ref in (("q", qo, rq), ("k", ko, rk)):
        x = got.float().cpu().numpy().astype(np.float64)
        err = np.abs(x - ref) - rel * np.abs(ref)
        assert err.max() <= 1e-12, (name, float(err.max()))
    for name, got, ref in (("g", g, rg), ("beta", beta, rb)):
        x = got.cpu().numpy().astype(np.float64)
        r = np.max(np.abs(x - ref) / np.maximum(np.abs(ref), 1e-30))
        report(f"prologue {io} {gate} {name}", max_rel=r)
        assert r <= 1e-5, (name, r)
    assert (g.cpu().numpy() < 0).all()


@pytest.mark.parametrize("B,T,H,Dk,io", [(1, 1, 1, 64, "bf16"), (2, 77, 3, 128, "bf16"), (1, 130, 2, 64, "fp32"),
                                         (4, 4096, 8, 128, "bf16")])
def test_channel_gate_prologue_matches_oracle(B, T, H, Dk, io):
    # one log-decay per key channel (the KDA gate layout): a and g shaped like q, dt_bias (H, Dk)
    q, k, _, b, A_log, _ = _raw(B, T, H, Dk, io, seed=B * 7 + T)
    rng = np.random.default_rng(T)
    a = rng.standard_normal((B, T, H, Dk), dtype=np.float32)
    dt = (np.float32(0.5) * rng.standard_normal((H, Dk), dtype=np.float32)).astype(np.float32)
    iot = torch.bfloat16 if io == "bf16" else torch.float32
    qo, ko, g, beta = gdn.prologue(_dev(q, iot), _dev(k, iot), _dev(a), _dev(b), _dev(A_log), _dev(dt),
                                   gate="gdn_channel")
    torch.cuda.synchronize()
    rq, rk, rg, rb = oracle.prologue(q, k, a, b, A_log, dt, gate="gdn_channel")
    assert tuple(g.shape) == (B, T, H, Dk)
    for name, got, ref in (("g", g, rg), ("beta", beta, rb)):
        x = got.cpu().numpy().astype(np.float64)
        r = np.max(np.abs(x - ref) / np.maximum(np.abs(ref), 1e-30))
        report(f"prologue {io} gdn_channel {name}", max_rel=r)
        assert r <= 1e-5, (name, r)
    rel = 2.0 ** -8 if io == "bf16" else 4e-7
    x = ko.float().cpu().numpy().astype(np.float64)
    assert (np.abs(x - rk) - rel * np.abs(rk)).max() <= 1e-12


def test_prologue_feeds_the_chunked_forward():
    B, T, H, Dk, Dv = 2, 257, 3, 128, 64
    q, k, a, b, A_log, dt = _raw(B, T, H, Dk, "bf16", seed=77)
    v = round_bf16(np.random.default_rng(78).standard_normal((B, T, H, Dv), dtype=np.float32))
    qo, ko, g, beta = gdn.prologue(_dev(q, torch.bfloat16), _dev(k, torch.bfloat16), _dev(a), _dev(b), _dev(A_log),
                                   _dev(dt))
    o, Sf = gdn.chunk_fwd(qo, ko, _dev(v, torch.bfloat16), g, beta)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.fwd(qo.float().cpu().numpy(), ko.float().cpu().numpy(), v, g.cpu().numpy(),
                              beta.cpu().numpy())
    eo = rel_rms(o.float().cpu().numpy(), o_ref.reshape(o.shape))
    es = rel_rms(Sf.cpu().numpy(), S_ref)
    report("prologue -> chunk_fwd", o_rel_rms=eo, S_rel_rms=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16


def test_channel_gate_prologue_feeds_the_kda_forward():
    # raw projections -> per-channel-gate prologue -> gdn_kda_chunk_fwd, against the
    # oracle run on the same (prologue-made) inputs
    B, T, H, Dk, Dv = 2, 200, 2, 128, 64
    q, k, _, b, A_log, _ = _raw(B, T, H, Dk, "bf16", seed=79)
    rng = np.random.default_rng(80)
    a = rng.standard_normal((B, T, H, Dk), dtype=np.float32)
    dt = (np.float32(0.5) * rng.standard_normal((H, Dk), dtype=np.float32)).astype(np.float32)
    v = round_bf16(rng.standard_normal((B, T, H, Dv), dtype=np.float32))
    qo, ko, g, beta = gdn.prologue(_dev(q, torch.bfloat16), _dev(k, torch.bfloat16), _dev(a), _dev(b), _dev(A_log),
                                   _dev(dt), gate="gdn_channel")
    o, Sf = gdn.kda_chunk_fwd(qo, ko, _dev(v, torch.bfloat16), g, beta)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.kda_fwd(qo.float().cpu().numpy(), ko.float().cpu().numpy(), v, g.cpu().numpy(),
                                  beta.cpu().numpy())
    eo = rel_rms(o.float().cpu().numpy(), o_ref.reshape(o.shape))
    es = rel_rms(Sf.cpu().numpy(), S_ref)
    report("prologue (channel gate) -> kda_chunk_fwd", o_rel_rms=eo, S_rel_rms=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16
