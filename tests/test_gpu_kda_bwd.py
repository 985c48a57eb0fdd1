"""GPU parity of the per-key-channel-decay backward (gdn_kda_chunk_bwd) against
the fp64 oracle's reverse mode ``oracle.kda_bwd`` (marked gpu).

Gradients of L = <o, dO> + <S_final, dS_final> with respect to q, k, v, the
per-channel log-decays g, beta and S0.  Tolerances as for the forward, each
gradient separately: max_rel <= 3e-4 for fp32 io, rel_rms <= 8e-3 for bf16 io
(the worst (sequence, head) is printed beside it).  Cases: both io dtypes and
head sizes, ragged tails, packed sequences with an empty and a one-token
sequence, an initial state and a final-state gradient, strong and slow decay,
run-to-run determinism, every head of the 4 x 4096 x 8 x 128 training shape
over its first 512 tokens, four of its (sequence, head) pairs over all 4096
tokens, and at full length the reduction to the scalar-gate backward (equal
decays on every channel; gdn_chunk_bwd is itself checked against the oracle).
"""
import numpy as np
import pytest
import torch

import gated_deltanet_chunked_gdn_amd as gdn
import oracle
from gated_deltanet_chunked_gdn_amd.workloads import WORKLOADS, Workload, generate
from oracle.compare import max_rel, rel_rms, worst_head_rel_rms
from _helpers import to_device, to_np, truncate

pytestmark = pytest.mark.gpu

FP32_TOL = 3e-4
BF16_TOL = 8e-3
GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


def _dsf(d, seed):
    w = d["workload"]
    N = len(d["cu_seqlens"]) - 1 if d["cu_seqlens"] is not None else w.B
    rng = np.random.default_rng(seed)
    return (0.1 * rng.standard_normal((N, w.H, w.Dk, w.Dv))).astype(np.float32)


def _run(d, t, dS_final):
    dsf = None if dS_final is None else torch.from_numpy(dS_final).cuda()
    out = gdn.kda_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dO"], S0=t.get("S0"), dS_final=dsf,
                            cu_seqlens=d["cu_seqlens"], scale=d["scale"])
    torch.cuda.synchronize()
    return {key: to_np(val) for key, val in out.items()}


def _oracle(d, dS_final):
    return oracle.kda_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["dO"], cu_seqlens=d["cu_seqlens"],
                          S0=d["S0"], dS_final=dS_final, scale=d["scale"])


def _check(d, got, ref, tag):
    for name in GRADS:
        out = got[name]
        r = ref[name].reshape(out.shape)
        assert np.isfinite(out).all(), (tag, name)
        if d["io"] == "fp32":
            e = max_rel(out, r)
            print(f"{tag} {name}: max_rel {e:.2e}", flush=True)
            assert e <= FP32_TOL, (tag, name)
        else:
            e = rel_rms(out, r)
            hw = worst_head_rel_rms(out, r, cu_seqlens=d["cu_seqlens"], token_major=name != "dS0")
            print(f"{tag} {name}: rel_rms {e:.2e} worst head {hw:.2e}", flush=True)
            assert e <= BF16_TOL, (tag, name)


CASES = [
    Workload("kdab_fp32_dk64", 2, 200, 2, 64, 64, io="fp32", qk="iid", gate="gdn_channel", s0_std=0.1,
             scale=0.7, with_dO=True, seed=71),
    Workload("kdab_fp32_dk128", 1, 130, 3, 128, 32, io="fp32", qk="norm_both", gate="gdn_channel",
             with_dO=True, seed=72),
    Workload("kdab_bf16_dk128", 2, 257, 2, 128, 128, io="bf16", qk="norm_both", gate="gdn_channel",
             s0_std=0.1, with_dO=True, seed=73),
    Workload("kdab_bf16_dk64_packed", 1, 300, 4, 64, 128, io="bf16", qk="norm_both", gate="gdn_channel",
             cu_seqlens=(0, 70, 70, 71, 300), s0_std=0.1, with_dO=True, seed=74),
    Workload("kdab_fp32_dk64_dv256_edges", 1, 200, 2, 64, 256, io="fp32", qk="norm_both", gate="gdn_channel",
             cu_seqlens=(0, 1, 65, 200), s0_std=0.1, scale=0.3, with_dO=True, seed=75),
    Workload("kdab_bf16_dk128_dv16_edges", 1, 130, 2, 128, 16, io="bf16", qk="iid", gate="gdn_channel",
             cu_seqlens=(0, 64, 65, 130), with_dO=True, seed=76),
    # d_v = 48: one full 32-column tile of the bf16 gradient kernel and a half one
    Workload("kdab_bf16_dk64_dv48", 2, 150, 2, 64, 48, io="bf16", qk="norm_both", gate="gdn_channel",
             s0_std=0.1, with_dO=True, seed=80),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_kda_bwd_matches_oracle(w):
    d = generate(w)
    dsf = _dsf(d, 7)
    _check(d, _run(d, to_device(d), dsf), _oracle(d, dsf), w.name)


@pytest.mark.parametrize("kind", ["strong", "slow", "edge"])
def test_kda_bwd_decay_extremes(kind):
    w = Workload(f"kdab_{kind}", 1, 200, 2, 128, 64, io="fp32", qk="norm_both", gate="gdn_channel",
                 s0_std=0.1, with_dO=True, seed=77)
    d = generate(w)
    rng = np.random.default_rng(78)
    shape = d["q"].shape
    if kind == "strong":
        # per-channel log-decays down to -5 per token; channel 0 of head 1 at -12, so
        # that head's chunks take the gradient kernel's pair-by-pair path (more than
        # 2^100 across half a 16-row block) and head 0's the products through the
        # middle row
        g = -5.0 / (1.0 + np.exp(-rng.standard_normal(shape)))
        g[:, :, 1, 0] = -12.0
    elif kind == "edge":
        # channel 0 of every head at -8.5 per token: 98.1 in log2 across half a 16-row
        # block, just inside the bound of the products through the middle row
        g = -4.0 / (1.0 + np.exp(-rng.standard_normal(shape)))
        g[..., 0] = -8.5
    else:
        g = -1e-3 * rng.random(shape)
    d["g"] = g.astype(np.float32)
    dsf = _dsf(d, 8)
    _check(d, _run(d, to_device(d), dsf), _oracle(d, dsf), w.name)


def test_kda_bwd_deterministic():
    d = generate(CASES[2])
    t = to_device(d)
    a = gdn.kda_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dO"], S0=t["S0"])
    b = gdn.kda_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dO"], S0=t["S0"])
    torch.cuda.synchronize()
    for name in GRADS:
        assert torch.equal(a[name], b[name]), name


def test_kda_bwd_training_shape_heads_first_512_tokens():
    # every (sequence, head) of the 4 x 4096 x 8 x 128 bf16 shape with per-channel
    # gates, over the first 512 tokens (eight chunks; the oracle keeps every state)
    w = WORKLOADS["kda_bf16"]
    d = generate(Workload(w.name, w.B, w.T, w.H, w.Dk, w.Dv, io=w.io, qk=w.qk, gate=w.gate, with_dO=True,
                          seed=w.seed))
    d = truncate(d, 512)
    _check(d, _run(d, to_device(d), None), _oracle(d, None), "kda_bf16[:512]")


def test_kda_bwd_training_shape_full_length_sampled_heads():
    # the whole 4 x 4096 x 8 x 128 bf16 backward with per-channel gates in one call;
    # (sequence, head) pairs are independent, so the oracle's reverse mode runs on
    # four of them over all 4096 tokens (about a second each).  Heads 0 of sequence
    # 2 and 6 of sequence 3 hold this workload's two chunks steeper than 2^100 across
    # half a 16-row block (pair-by-pair sums) beside many just inside that bound.
    w = WORKLOADS["kda_bf16"]
    d = generate(Workload(w.name, w.B, w.T, w.H, w.Dk, w.Dv, io=w.io, qk=w.qk, gate=w.gate, with_dO=True,
                          seed=w.seed))
    got = _run(d, to_device(d), None)

    def sl(x, n, h):
        return np.ascontiguousarray(x[n:n + 1, :, h:h + 1])

    for n, h in ((2, 0), (3, 6), (0, 3), (1, 5)):
        ref = oracle.kda_bwd(*(sl(d[key], n, h) for key in ("q", "k", "v", "g", "beta", "dO")), scale=d["scale"])
        for name in GRADS:
            out = got[name][n, :, h] if name != "dS0" else got[name][n, h]
            e = rel_rms(out, ref[name].reshape(out.shape))
            print(f"kda_bf16 full length (n={n}, h={h}) {name}: rel_rms {e:.2e}", flush=True)
            assert np.isfinite(out).all() and e <= BF16_TOL, (n, h, name)


def test_kda_bwd_full_length_equal_decays_is_the_scalar_gate_backward():
    # at the full 4 x 4096 x 8 x 128 shape: with one decay shared by every channel
    # the per-channel backward is the scalar-gate backward, and dg summed over the
    # channels is its dg (two independent kernel families, each within 8e-3 of the
    # oracle; their difference is held to the sum of the two bars)
    w = Workload("kdab_equal_full", 4, 4096, 8, 128, 128, io="bf16", qk="norm_both", gate="gdn", with_dO=True,
                 seed=79)
    d = generate(w)
    t = to_device(d)
    gk = t["g"][..., None].expand(*d["q"].shape).contiguous()
    a = gdn.kda_chunk_bwd(t["q"], t["k"], t["v"], gk, t["beta"], t["dO"], scale=d["scale"])
    b = gdn.chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dO"], scale=d["scale"])
    torch.cuda.synchronize()
    a["dg"] = a["dg"].sum(-1)
    for name in GRADS:
        x, y = to_np(a[name]), to_np(b[name])
        assert np.isfinite(x).all(), name
        e = rel_rms(x, y)
        print(f"equal decays, full length {name}: rel_rms against gdn_chunk_bwd {e:.2e}", flush=True)
        assert e <= 2 * BF16_TOL, name


@pytest.mark.parametrize("w", [CASES[2], CASES[3]], ids=lambda w: w.name)
def test_kda_retained_states_bit_identical(w):
    # gdn_kda_chunk_fwd_save gives gdn_kda_chunk_fwd's outputs bit for bit, and
    # gdn_kda_chunk_bwd_saved (twice on one buffer) gdn_kda_chunk_bwd's gradients
    d = generate(w)
    t = to_device(d)
    cu = d["cu_seqlens"]
    dsf = torch.from_numpy(_dsf(d, 9)).cuda()
    o_ref, sf_ref = gdn.kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=t.get("S0"), cu_seqlens=cu,
                                      scale=d["scale"])
    g_ref = gdn.kda_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dO"], S0=t.get("S0"), dS_final=dsf,
                              cu_seqlens=cu, scale=d["scale"])
    o, sf, saved = gdn.kda_chunk_fwd_save(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=t.get("S0"), cu_seqlens=cu,
                                          scale=d["scale"])
    for rep in range(2):
        got = gdn.kda_chunk_bwd_saved(t["q"], t["k"], t["v"], t["g"], t["beta"], t["dO"], saved, dS_final=dsf,
                                      cu_seqlens=cu, scale=d["scale"])
        torch.cuda.synchronize()
        for name in GRADS:
            assert torch.equal(got[name], g_ref[name]), (rep, name)
    assert torch.equal(o, o_ref) and torch.equal(sf, sf_ref)
