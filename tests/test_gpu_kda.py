"""GPU parity of the per-key-channel-decay forward (gdn_kda_chunk_fwd) against
the fp64 oracle ``oracle.kda_fwd`` (marked gpu).

Tolerances (each of o and S_final separately): max_rel <= 3e-4 for fp32 io,
rel_rms <= 8e-3 for bf16 io -- the bars of the scalar-gate path.  Cases: both io
dtypes and head sizes, ragged tails, packed sequences with an empty one, an
initial state, strong and slow per-channel decay, equal decays on every channel
(the scalar-gate recurrence), run-to-run determinism, and the 4 x 4096 x 8 x 128
training shape in the launch configuration bench.py times (every head).
"""
import numpy as np
import pytest
import torch

import gated_deltanet_chunked_gdn_amd as gdn
import oracle
from gated_deltanet_chunked_gdn_amd.workloads import WORKLOADS, Workload, generate
from oracle.compare import max_rel, rel_rms, worst_head_rel_rms
from _helpers import to_device, to_np

pytestmark = pytest.mark.gpu

FP32_TOL = 3e-4
BF16_TOL = 8e-3


def _run(d, t, G=1):
    cu = d["cu_seqlens"]
    o, Sf = gdn.kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=t.get("S0"),
                              cu_seqlens=cu, scale=d["scale"], num_segments=G)
    torch.cuda.synchronize()
    return to_np(o), to_np(Sf)


def _oracle(d):
    o, Sf = oracle.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu_seqlens"],
                           S0=d["S0"], scale=d["scale"])
    return o.reshape(d["v"].shape), Sf


def _check(d, got, ref, tag):
    (o, Sf), (o_ref, Sf_ref) = got, ref
    assert np.isfinite(o).all() and np.isfinite(Sf).all(), tag
    if d["io"] == "fp32":
        eo, es = max_rel(o, o_ref), max_rel(Sf, Sf_ref)
        print(f"{tag}: max_rel o {eo:.2e} S_final {es:.2e}")
        assert eo <= FP32_TOL and es <= FP32_TOL, tag
    else:
        eo, es = rel_rms(o, o_ref), rel_rms(Sf, Sf_ref)
        print(f"{tag}: rel_rms o {eo:.2e} S_final {es:.2e}")
        assert eo <= BF16_TOL and es <= BF16_TOL, tag


CASES = [
    Workload("kda_fp32_dk64", 2, 200, 2, 64, 64, io="fp32", qk="iid", gate="gdn_channel", s0_std=0.1,
             scale=0.7, seed=51),
    Workload("kda_fp32_dk128", 1, 130, 3, 128, 32, io="fp32", qk="norm_both", gate="gdn_channel", seed=52),
    Workload("kda_bf16_dk128", 2, 257, 2, 128, 128, io="bf16", qk="norm_both", gate="gdn_channel",
             s0_std=0.1, seed=53),
    Workload("kda_bf16_dk64_dv128", 1, 300, 4, 64, 128, io="bf16", qk="norm_both", gate="gdn_channel",
             cu_seqlens=(0, 70, 70, 300), s0_std=0.1, seed=54),
    # a one-token sequence, one of exactly one chunk, one with a ragged tail; the widest d_v
    Workload("kda_fp32_dk64_dv256_edges", 1, 200, 2, 64, 256, io="fp32", qk="norm_both", gate="gdn_channel",
             cu_seqlens=(0, 1, 65, 200), s0_std=0.1, scale=0.3, seed=58),
    Workload("kda_bf16_dk128_dv16_edges", 1, 130, 2, 128, 16, io="bf16", qk="iid", gate="gdn_channel",
             cu_seqlens=(0, 64, 65, 130), seed=59),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_kda_matches_oracle(w):
    d = generate(w)
    _check(d, _run(d, to_device(d)), _oracle(d), w.name)


@pytest.mark.parametrize("kind", ["strong", "slow", "steep", "bounded", "edge"])
def test_kda_decay_extremes(kind):
    # The preparation forms the diagonal 16x16 blocks of A and P as products through
    # their middle row while no channel decays by more than 2^-100 across either half
    # of a block, and pair by pair otherwise: "steep" takes the pair-by-pair path in
    # every chunk, "bounded" (up to ~2^-87 per whole block) never does, "strong"
    # mixes both (head 0 through the products, head 1 pair by pair); "edge" sits just
    # inside the bound (factors up to ~2^98; the products' discarded entries above
    # the diagonal overflow).
    w = Workload(f"kda_{kind}", 1, 260, 2, 128, 64, io="bf16", qk="norm_both", gate="gdn_channel",
                 s0_std=0.1, seed=55)
    d = generate(w)
    rng = np.random.default_rng(56)
    shape = d["q"].shape
    if kind == "strong":
        # per-channel log-decays down to -5 per token: exp(gamma) underflows within a
        # chunk; channel 0 of head 1 decays by 12 per token (96 nats, 138.5 in log2,
        # across half a block)
        g = -5.0 / (1.0 + np.exp(-rng.standard_normal(shape)))
        g[:, :, 1, 0] = -12.0
        d["g"] = g.astype(np.float32)
    elif kind == "steep":
        # channel 0 of every head decays by 12 per token
        g = -4.0 / (1.0 + np.exp(-rng.standard_normal(shape)))
        g[..., 0] = -12.0
        d["g"] = g.astype(np.float32)
    elif kind == "edge":
        # channel 0 of every head decays by 8.5 per token: 68 nats (98.1 in log2) across half a block
        g = -4.0 / (1.0 + np.exp(-rng.standard_normal(shape)))
        g[..., 0] = -8.5
        d["g"] = g.astype(np.float32)
    elif kind == "bounded":
        # at most 4 per token: at most 60 nats (87 in log2) across a block
        d["g"] = (-4.0 / (1.0 + np.exp(-3.0 * rng.standard_normal(shape)))).astype(np.float32)
    else:
        d["g"] = (-1e-3 * rng.random(shape)).astype(np.float32)
    _check(d, _run(d, to_device(d)), _oracle(d), w.name)


def test_kda_equal_channel_decays_is_the_scalar_gate_recurrence():
    w = Workload("kda_equal", 2, 190, 2, 128, 128, io="bf16", qk="norm_both", gate="gdn", s0_std=0.1,
                 seed=57)
    d = generate(w)
    t = to_device(d)
    t["g"] = t["g"][..., None].expand(*d["q"].shape).contiguous()
    got = _run(d, t)
    o_ref, Sf_ref = oracle.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], S0=d["S0"], scale=d["scale"])
    _check(d, got, (o_ref.reshape(d["v"].shape), Sf_ref), "equal channel decays vs scalar-gate oracle")


def test_kda_deterministic():
    d = generate(CASES[2])
    t = to_device(d)
    a = gdn.kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=t["S0"])
    b = gdn.kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], S0=t["S0"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_kda_training_shape_every_head():
    # the 4 x 4096 x 8 x 128 bf16 shape with per-channel gates, as bench.py runs it;
    # the oracle recomputes all 32 (sequence, head) pairs in full (about 10 s)
    w = WORKLOADS["kda_bf16"]
    d = generate(w)
    t = to_device(d)
    o, Sf = gdn.kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=w.scale)
    torch.cuda.synchronize()
    o, Sf = to_np(o), to_np(Sf)
    assert np.isfinite(o).all() and np.isfinite(Sf).all()
    o_ref, Sf_ref = oracle.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=w.scale)
    o_ref = o_ref.reshape(o.shape)
    eo, es = rel_rms(o, o_ref), rel_rms(Sf, Sf_ref)
    ho = worst_head_rel_rms(o, o_ref)
    hs = worst_head_rel_rms(Sf, Sf_ref, token_major=False)
    print(f"kda_bf16: rel_rms o {eo:.2e} S_final {es:.2e}; worst head o {ho:.2e} S_final {hs:.2e}")
    assert eo <= BF16_TOL and es <= BF16_TOL
    assert ho <= BF16_TOL and hs <= BF16_TOL


# ---- segment split (cuLA issue #126: "Summary", "Minimal public reproduction") ----

SEG_CASES = [
    (Workload("kda_seg_fp32", 2, 700, 2, 64, 64, io="fp32", qk="norm_both", gate="gdn_channel", s0_std=0.3,
              seed=61), 4),
    (Workload("kda_seg_bf16", 1, 2000, 2, 128, 48, io="bf16", qk="norm_both", gate="gdn_channel",
              cu_seqlens=(0, 64, 64, 129, 1500, 2000), s0_std=0.2, seed=62), 16),
    (Workload("kda_seg_bf16_dk64", 2, 1300, 2, 64, 128, io="bf16", qk="norm_both", gate="channel_slow",
              s0_std=0.1, seed=63), 8),
    (Workload("kda_seg_few_chunks", 3, 130, 2, 128, 64, io="bf16", qk="norm_both", gate="gdn_channel",
              s0_std=0.1, seed=64), 16),
]


@pytest.mark.parametrize("w,G", SEG_CASES, ids=lambda x: x.name if hasattr(x, "name") else f"G{x}")
def test_kda_segments_match_oracle_and_serial(w, G):
    d = generate(w)
    t = to_device(d)
    got = _run(d, t, G)
    _check(d, got, _oracle(d), f"{w.name} G={G}")
    # G = 2 and the rows of the first two segments are computed exactly as in the serial pass
    one, two = _run(d, t, 1), _run(d, t, 2)
    assert np.array_equal(two[0], one[0]) and np.array_equal(two[1], one[1])
    if d["cu_seqlens"] is None:
        L = -(-(-(-w.T // 64)) // G)
        rows = min(2 * L * 64, w.T)
        assert np.array_equal(got[0][:, :rows], one[0][:, :rows])


@pytest.fixture(scope="module")
def kda_long():
    d = generate(WORKLOADS["kda_long_bf16"])
    t = to_device(d)
    o_ref, S_ref = _oracle(d)
    one = _run(d, t, 1)
    return d, t, o_ref, S_ref, one


def test_kda_long_serial(kda_long):
    d, t, o_ref, S_ref, (o1, S1) = kda_long
    win = [rel_rms(o1[:, 8192 * i:8192 * (i + 1)], o_ref[:, 8192 * i:8192 * (i + 1)]) for i in range(8)]
    es = rel_rms(S1, S_ref)
    print("kda_long G=1: windows " + " ".join(f"{e:.2e}" for e in win) + f"; S_final {es:.2e}")
    assert max(win) <= BF16_TOL and es <= BF16_TOL


@pytest.mark.parametrize("G", [2, 4, 8, 16])
def test_kda_long_segments_per_window(kda_long, G):
    """Per-8K-window rel-L2 against the oracle and against the serial pass (the
    windows of the cuLA issue #126 page's reproduction)."""
    d, t, o_ref, S_ref, (o1, S1) = kda_long
    o, Sf = _run(d, t, G)
    win = [rel_rms(o[:, 8192 * i:8192 * (i + 1)], o_ref[:, 8192 * i:8192 * (i + 1)]) for i in range(8)]
    win1 = [rel_rms(o[:, 8192 * i:8192 * (i + 1)], o1[:, 8192 * i:8192 * (i + 1)]) for i in range(8)]
    es, es1 = rel_rms(Sf, S_ref), rel_rms(Sf, S1)
    print(f"kda_long G={G}: windows vs oracle " + " ".join(f"{e:.2e}" for e in win)
          + "; vs serial " + " ".join(f"{e:.2e}" for e in win1) + f"; S_final {es:.2e} (vs serial {es1:.2e})")
    assert max(win) <= BF16_TOL and es <= BF16_TOL
    assert max(win1) <= BF16_TOL and es1 <= BF16_TOL
    L = -(-1024 // G)
    rows = min(2 * L * 64, 65536)
    assert np.array_equal(o[:, :rows], o1[:, :rows])
    if G == 2:
        assert np.array_equal(o, o1) and np.array_equal(Sf, S1)
