"""Pins of the oracle's input prologue (CPU only): invariants of the L2
normalisation, closed forms of the gates at points where they have exact values,
their asymptotics and ranges, and agreement with the workload generator's own
float32 formulas.  Gate formulas: "Research Sprint Day 2", "Building some
intuition" (g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b), doubled under
negative eigenvalues); normalisation before the cast: fla issue #1550 page,
"Proposed scope"; the bounded gates -5 sigmoid(a) of that page's workload.
"""
import math

import numpy as np

import oracle
from gated_deltanet_chunked_gdn_amd import workloads


def _draw(seed=5, shape=(2, 7, 3, 64)):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(shape)
    k = rng.standard_normal(shape)
    a = rng.standard_normal(shape[:3])
    b = rng.standard_normal(shape[:3])
    A_log = rng.uniform(0.0, 1.5, size=shape[2])
    dt = 0.5 * rng.standard_normal(shape[2])
    return q, k, a, b, A_log, dt


def test_normalised_rows_have_unit_norm_and_keep_direction():
    q, k, a, b, A_log, dt = _draw()
    qn, kn, _, _ = oracle.prologue(q, k, a, b, A_log, dt)
    assert np.allclose(np.linalg.norm(qn, axis=-1), 1.0, atol=1e-14)
    assert np.allclose(np.linalg.norm(kn, axis=-1), 1.0, atol=1e-14)
    # positive multiples of the input: <q_n, q> = ||q||
    assert np.allclose(np.sum(qn * q, axis=-1), np.linalg.norm(q, axis=-1), rtol=1e-13)


def test_normalisation_is_scale_invariant():
    q, k, a, b, A_log, dt = _draw()
    q1, k1, _, _ = oracle.prologue(q, k, a, b, A_log, dt)
    q2, k2, _, _ = oracle.prologue(3.5 * q, 0.01 * k, a, b, A_log, dt)
    assert np.allclose(q1, q2, atol=1e-15) and np.allclose(k1, k2, atol=1e-15)


def test_zero_row_stays_zero():
    q = np.zeros((1, 1, 1, 64))
    qn, kn, _, _ = oracle.prologue(q, q, np.zeros((1, 1, 1)), np.zeros((1, 1, 1)), np.zeros(1), np.zeros(1))
    assert np.all(qn == 0.0) and np.all(kn == 0.0)


def test_beta_closed_forms():
    H = 1
    b = np.array([0.0, math.log(3.0), -math.log(3.0)]).reshape(1, 3, 1)
    z = np.zeros((1, 3, 1, 64))
    _, _, _, beta = oracle.prologue(z, z, np.zeros((1, 3, 1)), b, np.zeros(H), np.zeros(H))
    assert np.allclose(beta.ravel(), [0.5, 0.75, 0.25], atol=1e-15)
    _, _, _, beta2 = oracle.prologue(z, z, np.zeros((1, 3, 1)), b, np.zeros(H), np.zeros(H), allow_neg_eigval=True)
    assert np.allclose(beta2.ravel(), [1.0, 1.5, 0.5], atol=1e-15)


def test_gdn_gate_closed_forms_and_asymptotics():
    A_log = np.array([0.0, 0.7, 1.5])
    dt = np.array([0.3, -0.2, 1.1])
    # a + dt_bias = 0: softplus = ln 2; a + dt_bias = ln(e - 1): softplus = 1;
    # a + dt_bias = 40: softplus = 40 (+ e^-40); a + dt_bias = -40: softplus = e^-40
    xs = np.array([0.0, math.log(math.e - 1.0), 40.0, -40.0])
    a = (xs[:, None] - dt[None, :]).reshape(1, 4, 3)
    z = np.zeros((1, 4, 3, 64))
    _, _, g, _ = oracle.prologue(z, z, a, np.zeros((1, 4, 3)), A_log, dt)
    e = np.exp(A_log)
    assert np.allclose(g[0, 0], -e * math.log(2.0), rtol=1e-14)
    assert np.allclose(g[0, 1], -e, rtol=1e-14)
    assert np.allclose(g[0, 2], -e * 40.0, rtol=1e-14)
    assert np.allclose(g[0, 3], -e * math.exp(-40.0), rtol=1e-12)
    assert np.all(g < 0.0)


def test_bounded_gate_closed_forms_and_range():
    a = np.array([0.0, math.log(3.0), -math.log(3.0), 50.0, -50.0]).reshape(1, 5, 1)
    z = np.zeros((1, 5, 1, 64))
    _, _, g, _ = oracle.prologue(z, z, a, np.zeros((1, 5, 1)), gate="bounded5")
    assert np.allclose(g.ravel()[:3], [-2.5, -3.75, -1.25], atol=1e-14)
    assert -5.0 <= g.min() and g.max() < 0.0


def test_gates_and_norms_agree_with_the_generators_float32_formulas():
    q, k, a, b, A_log, dt = _draw(seed=9)
    f = np.float32
    qn, kn, g, beta = oracle.prologue(q.astype(f), k.astype(f), a.astype(f), b.astype(f), A_log.astype(f),
                                      dt.astype(f))
    g32 = -np.exp(A_log.astype(f)) * workloads._softplus(a.astype(f) + dt.astype(f))
    assert np.allclose(g, g32, rtol=2e-6, atol=0)
    assert np.allclose(beta, workloads._sigmoid(b.astype(f)), rtol=2e-6, atol=0)
    assert np.allclose(qn, workloads._normalize(q.astype(f)), rtol=0, atol=2e-7)
    g5 = oracle.prologue(q, k, a.astype(f), b, gate="bounded5")[2]
    assert np.allclose(g5, f(-5.0) * workloads._sigmoid(a.astype(f)), rtol=2e-6, atol=0)


def test_channel_gate_closed_forms_and_reduction_to_the_head_gate():
    # per key channel: the same closed forms channel by channel, and with a and
    # dt_bias equal on every channel it is the head gate repeated over channels
    A_log = np.array([0.0, 0.7, 1.5])
    xs = np.array([0.0, math.log(math.e - 1.0), 40.0, -40.0])
    dt = 0.25 * np.arange(3 * 8).reshape(3, 8) - 2.0            # (H, Dk)
    a = (xs[:, None, None] - dt[None, :, :]).reshape(1, 4, 3, 8)
    z = np.zeros((1, 4, 3, 8))
    _, _, g, _ = oracle.prologue(z, z, a, np.zeros((1, 4, 3)), A_log, dt, gate="gdn_channel")
    e = np.exp(A_log)[:, None]
    assert g.shape == (1, 4, 3, 8)
    assert np.allclose(g[0, 0], -e * math.log(2.0), rtol=1e-14)
    assert np.allclose(g[0, 1], -e, rtol=1e-14)
    assert np.allclose(g[0, 2], -e * 40.0, rtol=1e-14)
    assert np.allclose(g[0, 3], -e * math.exp(-40.0), rtol=1e-12)
    q, k, a1, b, A_log1, dt1 = _draw(seed=11, shape=(2, 5, 3, 16))
    _, _, g_head, _ = oracle.prologue(q, k, a1, b, A_log1, dt1)
    _, _, g_chan, _ = oracle.prologue(q, k, np.repeat(a1[..., None], 16, axis=-1), b, A_log1,
                                      np.repeat(dt1[:, None], 16, axis=-1), gate="gdn_channel")
    assert np.allclose(g_chan, g_head[..., None], rtol=0, atol=0)
    # the seeded per-channel generator of the KDA workload draws the same formula in float32
    f = np.float32
    w = workloads.WORKLOADS["kda_bf16"].with_(B=1, T=16, H=2, Dk=8, Dv=8)
    rng = np.random.default_rng(w.seed)
    for _ in range(3):   # q_raw, k_raw, v, as the generator draws them
        rng.standard_normal((1, 16, 2, 8), dtype=f)
    a_g = rng.standard_normal((1, 16, 2, 8), dtype=f)
    A_log_g = rng.uniform(0.0, 1.5, size=(2,)).astype(f)
    dt_g = (f(0.5) * rng.standard_normal((2, 8), dtype=f)).astype(f)
    g_ref = oracle.prologue(np.zeros((1, 16, 2, 8)), np.zeros((1, 16, 2, 8)), a_g, np.zeros((1, 16, 2)), A_log_g,
                            dt_g, gate="gdn_channel")[2]
    assert np.allclose(workloads.generate(w)["g"], g_ref, rtol=3e-6, atol=0)
