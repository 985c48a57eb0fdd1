"""Pins of the CPU fp64 oracle to facts other than itself (CPU only).

Each test checks the oracle against something the pages or mathematics fix:
a hand-worked example, the closed form and the fused form printed on the Day-2
page, a special case that is a textbook filter (scipy.signal.lfilter), invariants
of the delta rule, and central finite differences for the backward pass.  They
are chosen so that a dropped term, a wrong sign, the wrong order of forget/read/
write, an output read before the write, or a transposed state all fail.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.signal

import oracle
from oracle.compare import max_rel, rel_rms

RNG = np.random.default_rng(12345)


def _rand_inputs(B, T, H, Dk, Dv, rng, beta_hi=1.0, gscale=0.3):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    g = -gscale * rng.random((B, T, H))
    beta = beta_hi * rng.random((B, T, H))
    return q, k, v, g, beta


# ----------------------------------------------------------------------------------------
# Hand-worked example (tests/golden/worked_example_dk2.txt)
# ----------------------------------------------------------------------------------------
def test_hand_worked_example(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "worked_example_dk2.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            left, o_exp, s_exp = line.split("|")
            rows.append(([float(x) for x in left.split()[1:]], float(o_exp),
                         [float(x) for x in s_exp.split()]))
    T = len(rows)
    k = np.array([r[0][0:2] for r in rows]).reshape(1, T, 1, 2)
    v = np.array([r[0][2] for r in rows]).reshape(1, T, 1, 1)
    q = np.array([r[0][3:5] for r in rows]).reshape(1, T, 1, 2)
    g = np.array([r[0][5] for r in rows]).reshape(1, T, 1)
    beta = np.array([r[0][6] for r in rows]).reshape(1, T, 1)
    o_exp = np.array([r[1] for r in rows])
    for t in range(1, T + 1):  # the state after every prefix
        o, S = oracle.fwd(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t])
        np.testing.assert_allclose(S[0, 0, :, 0], rows[t - 1][2], rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[0, :, 0, 0], o_exp, rtol=0, atol=1e-14)
    # the output is linear in scale
    o2, _ = oracle.fwd(q, k, v, g, beta, scale=0.5)
    np.testing.assert_allclose(o2[0, :, 0, 0], 0.5 * o_exp, rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------------------
# Closed form of the Day-2 page ("Building some intuition"):
#   S'_t = S'_{t-1} (alpha_t (I - beta_t k_t k_t^T)) + beta_t v_t k_t^T
# with S' the d_v x d_k state (the transpose of the oracle's d_k x d_v S), and its
# unrolled sum over explicit transition matrices.
# ----------------------------------------------------------------------------------------
def _closed_form_states(q, k, v, g, beta, S0=None):
    """Per (b, h): states S'_t (d_v x d_k) by explicit d_k x d_k transitions."""
    B, T, H, Dk = k.shape
    Dv = v.shape[-1]
    states = np.zeros((B, T, H, Dv, Dk))
    for b in range(B):
        for h in range(H):
            Sp = np.zeros((Dv, Dk)) if S0 is None else S0[b, h].T.copy()
            for t in range(T):
                kk = k[b, t, h][:, None]
                M = math.exp(g[b, t, h]) * (np.eye(Dk) - beta[b, t, h] * (kk @ kk.T))
                Sp = Sp @ M + beta[b, t, h] * v[b, t, h][:, None] @ kk.T
                states[b, t, h] = Sp
    return states


def _unrolled_final(k, v, g, beta, S0, b, h):
    """S'_T = S'_0 Phi(0,T) + sum_t beta_t v_t k_t^T Phi(t,T), Phi(t,T) = M_{t+1} ... M_T."""
    T, Dk = k.shape[1], k.shape[3]
    Ms = []
    for t in range(T):
        kk = k[b, t, h][:, None]
        Ms.append(math.exp(g[b, t, h]) * (np.eye(Dk) - beta[b, t, h] * (kk @ kk.T)))
    total = S0[b, h].T @ np.linalg.multi_dot([np.eye(Dk)] + Ms + [np.eye(Dk)])
    for t in range(T):
        Phi = np.eye(Dk)
        for s in range(t + 1, T):
            Phi = Phi @ Ms[s]
        total = total + beta[b, t, h] * (v[b, t, h][:, None] @ k[b, t, h][None, :]) @ Phi
    return total


@pytest.mark.parametrize("Dk,Dv,T", [(4, 3, 9), (8, 8, 16), (3, 5, 1)])
def test_closed_form_transition(Dk, Dv, T):
    rng = np.random.default_rng(Dk * 100 + Dv * 10 + T)
    q, k, v, g, beta = _rand_inputs(2, T, 2, Dk, Dv, rng, beta_hi=1.9)
    S0 = 0.3 * rng.standard_normal((2, 2, Dk, Dv))
    o, Sf = oracle.fwd(q, k, v, g, beta, S0=S0, scale=0.7)
    st = _closed_form_states(q, k, v, g, beta, S0=S0)
    # o_t = scale * S_t^T q_t = scale * S'_t q_t
    o_cf = 0.7 * np.einsum("bthvk,bthk->bthv", st, q)
    assert rel_rms(o, o_cf) < 1e-13
    assert rel_rms(Sf, np.swapaxes(st[:, -1], -1, -2)) < 1e-13
    for b in range(2):
        for h in range(2):
            unrolled = _unrolled_final(k, v, g, beta, S0, b, h)
            assert rel_rms(Sf[b, h], unrolled.T) < 1e-13


def test_fused_form():
    """Day-2 page, "FLOPs per token": S'_t = a S'_{t-1} + (b v - a b S'_{t-1} k) k^T."""
    rng = np.random.default_rng(7)
    B, T, H, Dk, Dv = 1, 40, 3, 6, 7
    q, k, v, g, beta = _rand_inputs(B, T, H, Dk, Dv, rng, beta_hi=1.5)
    o, Sf = oracle.fwd(q, k, v, g, beta)
    for h in range(H):
        Sp = np.zeros((Dv, Dk))
        for t in range(T):
            a, bb = math.exp(g[0, t, h]), beta[0, t, h]
            kk = k[0, t, h]
            Sp = a * Sp + np.outer(bb * v[0, t, h] - a * bb * (Sp @ kk), kk)
            np.testing.assert_allclose(o[0, t, h], Sp @ q[0, t, h], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(Sf[0, h], Sp.T, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------------------
# d_k = d_v = 1, k = 1: s_t = alpha_t (1 - beta_t) s_{t-1} + beta_t v_t -- a first-order
# IIR filter (exponential moving average when alpha = 1), i.e. scipy.signal.lfilter.
# ----------------------------------------------------------------------------------------
@pytest.mark.parametrize("alpha,beta", [(1.0, 0.25), (0.9, 0.5), (0.7, 1.6)])
def test_scalar_case_is_iir_filter(alpha, beta):
    rng = np.random.default_rng(3)
    T = 300
    v = rng.standard_normal(T)
    qv = rng.standard_normal(T)
    s_ref = scipy.signal.lfilter([beta], [1.0, -alpha * (1.0 - beta)], v)
    o, Sf = oracle.fwd(qv.reshape(1, T, 1, 1), np.ones((1, T, 1, 1)), v.reshape(1, T, 1, 1),
                       np.full((1, T, 1), math.log(alpha)), np.full((1, T, 1), beta),
                       scale=1.3)
    np.testing.assert_allclose(o[0, :, 0, 0], 1.3 * qv * s_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Sf[0, 0, 0, 0], s_ref[-1], rtol=1e-12)


# ----------------------------------------------------------------------------------------
# Invariants of the delta rule
# ----------------------------------------------------------------------------------------
def test_beta_zero_only_decays():
    rng = np.random.default_rng(11)
    B, T, H, Dk, Dv = 2, 33, 2, 5, 4
    q, k, v, g, _ = _rand_inputs(B, T, H, Dk, Dv, rng)
    S0 = rng.standard_normal((B, H, Dk, Dv))
    o, Sf = oracle.fwd(q, k, v, g, np.zeros((B, T, H)), S0=S0, scale=0.9)
    Gam = np.exp(np.cumsum(g, axis=1))  # (B, T, H)
    np.testing.assert_allclose(Sf, Gam[:, -1][:, :, None, None] * S0, rtol=1e-13, atol=1e-15)
    o_exp = 0.9 * Gam[..., None] * np.einsum("bhkv,bthk->bthv", S0, q)
    np.testing.assert_allclose(o, o_exp, rtol=1e-12, atol=1e-14)


def test_orthonormal_keys_store_values_exactly():
    rng = np.random.default_rng(5)
    Dk, Dv, m = 8, 6, 8
    Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
    k = Qm.T[:m].reshape(1, m, 1, Dk)  # orthonormal rows
    v = rng.standard_normal((1, m, 1, Dv))
    o, Sf = oracle.fwd(np.zeros((1, m, 1, Dk)), k, v, np.zeros((1, m, 1)), np.ones((1, m, 1)))
    np.testing.assert_allclose(Sf[0, 0], k[0, :, 0].T @ v[0, :, 0], atol=1e-14)
    np.testing.assert_allclose(k[0, :, 0] @ Sf[0, 0], v[0, :, 0], atol=1e-14)


def test_unit_beta_replaces_the_value_under_the_key():
    """beta_t = 1, |k_t| = 1, any history: after token t, S^T k_t = v_t (read after write)."""
    rng = np.random.default_rng(8)
    B, T, H, Dk, Dv = 1, 50, 2, 7, 5
    _, k, v, g, beta = _rand_inputs(B, T, H, Dk, Dv, rng, beta_hi=1.8)
    beta[:, 1::3] = 1.0
    S0 = rng.standard_normal((B, H, Dk, Dv))
    o, _ = oracle.fwd(k.copy(), k, v, g, beta, S0=S0)  # q_t = k_t
    np.testing.assert_allclose(o[:, 1::3], v[:, 1::3], atol=1e-12)
    assert np.max(np.abs(o[:, 0::3] - v[:, 0::3])) > 1e-3  # beta != 1 does not replace


def test_linearity_in_v_and_S0_and_homogeneity():
    rng = np.random.default_rng(9)
    B, T, H, Dk, Dv = 1, 20, 2, 4, 3
    q, k, v1, g, beta = _rand_inputs(B, T, H, Dk, Dv, rng, beta_hi=1.9)
    v2 = rng.standard_normal(v1.shape)
    S1, S2 = rng.standard_normal((2, B, H, Dk, Dv))
    a, b = 0.7, -1.3
    o1, F1 = oracle.fwd(q, k, v1, g, beta, S0=S1)
    o2, F2 = oracle.fwd(q, k, v2, g, beta, S0=S2)
    o3, F3 = oracle.fwd(q, k, a * v1 + b * v2, g, beta, S0=a * S1 + b * S2)
    np.testing.assert_allclose(o3, a * o1 + b * o2, atol=1e-12)
    np.testing.assert_allclose(F3, a * F1 + b * F2, atol=1e-12)
    o4, _ = oracle.fwd(2.5 * q, k, v1, g, beta, S0=S1, scale=0.4)
    np.testing.assert_allclose(o4, o1, atol=1e-12)


def test_non_expansive_bound():
    """|k|=1, beta in (0,2): ||I - beta k k^T||_2 <= 1, so ||S_t|| <= a_t ||S_{t-1}|| + beta_t ||v_t||."""
    rng = np.random.default_rng(10)
    B, T, H, Dk, Dv = 1, 60, 1, 6, 4
    q, k, v, g, beta = _rand_inputs(B, T, H, Dk, Dv, rng, beta_hi=1.99)
    S0 = rng.standard_normal((B, H, Dk, Dv))
    prev = np.linalg.norm(S0[0, 0], 2)
    for t in range(1, T + 1):
        _, S = oracle.fwd(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], S0=S0)
        cur = np.linalg.norm(S[0, 0], 2)
        bound = math.exp(g[0, t - 1, 0]) * prev + beta[0, t - 1, 0] * np.linalg.norm(v[0, t - 1, 0])
        assert cur <= bound * (1 + 1e-12)
        prev = cur


def test_columns_of_the_state_are_independent():
    rng = np.random.default_rng(13)
    q, k, v, g, beta = _rand_inputs(1, 30, 1, 5, 6, rng)
    o1, F1 = oracle.fwd(q, k, v, g, beta)
    v2 = v.copy()
    v2[..., 2] += 1.0
    o2, F2 = oracle.fwd(q, k, v2, g, beta)
    others = [0, 1, 3, 4, 5]
    np.testing.assert_array_equal(o1[..., others], o2[..., others])
    np.testing.assert_array_equal(F1[..., others], F2[..., others])
    assert np.max(np.abs(o1[..., 2] - o2[..., 2])) > 1e-3


def test_packed_equals_separate_sequences_and_resume():
    rng = np.random.default_rng(14)
    H, Dk, Dv = 2, 5, 4
    lens = [7, 0, 19, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    Tt = int(cu[-1])
    q, k, v, g, beta = (x[0] for x in _rand_inputs(1, Tt, H, Dk, Dv, rng))
    S0 = rng.standard_normal((len(lens), H, Dk, Dv))
    o, Sf = oracle.fwd(q, k, v, g, beta, cu_seqlens=cu, S0=S0, scale=0.8)
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        if lens[n] == 0:
            np.testing.assert_array_equal(Sf[n], S0[n])
            continue
        o1, F1 = oracle.fwd(q[None, sl], k[None, sl], v[None, sl], g[None, sl], beta[None, sl],
                            S0=S0[n:n + 1], scale=0.8)
        np.testing.assert_array_equal(o[sl], o1[0])
        np.testing.assert_array_equal(Sf[n], F1[0])
    # resume: run 19 tokens as 11 + 8
    sl = slice(cu[2], cu[3])
    qq, kk, vv, gg, bb = (x[None, sl] for x in (q, k, v, g, beta))
    oa, Fa = oracle.fwd(qq[:, :11], kk[:, :11], vv[:, :11], gg[:, :11], bb[:, :11], S0=S0[2:3], scale=0.8)
    ob, Fb = oracle.fwd(qq[:, 11:], kk[:, 11:], vv[:, 11:], gg[:, 11:], bb[:, 11:], S0=Fa, scale=0.8)
    np.testing.assert_array_equal(np.concatenate([oa, ob], axis=1)[0], o[sl])
    np.testing.assert_array_equal(Fb[0], Sf[2])


def test_thread_count_does_not_change_bits():
    rng = np.random.default_rng(15)
    q, k, v, g, beta = _rand_inputs(2, 40, 3, 8, 16, rng)
    a = oracle.fwd(q, k, v, g, beta, nthreads=1)
    b = oracle.fwd(q, k, v, g, beta, nthreads=7)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_bad_cu_seqlens_rejected():
    q = np.zeros((5, 1, 2))
    with pytest.raises(ValueError):
        oracle.fwd(q, q, q, np.zeros((5, 1)), np.zeros((5, 1)), cu_seqlens=[0, 3, 2, 5])


# ----------------------------------------------------------------------------------------
# Backward: central finite differences of L = <o, dO> + <S_final, dS_final>
# ----------------------------------------------------------------------------------------
def _loss(inp, dO, dSf, scale, cu=None):
    o, Sf = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], S0=inp["S0"],
                       scale=scale, cu_seqlens=cu)
    return float(np.sum(o * dO) + np.sum(Sf * dSf))


@pytest.mark.parametrize("packed", [False, True])
def test_backward_matches_finite_differences(packed):
    rng = np.random.default_rng(21)
    B, T, H, Dk, Dv = (1, 13, 2, 4, 3) if packed else (2, 9, 2, 4, 3)
    q, k, v, g, beta = _rand_inputs(B, T, H, Dk, Dv, rng, beta_hi=1.8)
    cu = np.array([0, 5, 13]) if packed else None
    N = 2
    inp = {"q": q, "k": k, "v": v, "g": g, "beta": beta,
           "S0": 0.5 * rng.standard_normal((N, H, Dk, Dv))}
    if packed:
        for name in ("q", "k", "v", "g", "beta"):
            inp[name] = inp[name][0]
    dO = rng.standard_normal(inp["v"].shape)
    dSf = rng.standard_normal((N, H, Dk, Dv))
    scale = 0.6
    grads = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], dO, cu_seqlens=cu,
                       S0=inp["S0"], dS_final=dSf, scale=scale)
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "S0": "dS0"}
    h = 1e-6
    for name, gname in names.items():
        x = inp[name]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            orig = x[idx]
            x[idx] = orig + h
            lp = _loss(inp, dO, dSf, scale, cu)
            x[idx] = orig - h
            lm = _loss(inp, dO, dSf, scale, cu)
            x[idx] = orig
            fd[idx] = (lp - lm) / (2 * h)
        err = max_rel(grads[gname].reshape(fd.shape), fd)
        assert err < 1e-7, (gname, err)


def test_backward_beta_zero_closed_forms():
    """beta = 0: o_t = scale G_t S0^T q_t, so dv = 0, dbeta-free state and
    dS0 = scale sum_t G_t q_t dO_t^T + G_T dS_final, dq_t = scale G_t S0 dO_t."""
    rng = np.random.default_rng(22)
    B, T, H, Dk, Dv = 1, 17, 2, 5, 4
    q, k, v, g, _ = _rand_inputs(B, T, H, Dk, Dv, rng)
    beta = np.zeros((B, T, H))
    S0 = rng.standard_normal((B, H, Dk, Dv))
    dO = rng.standard_normal((B, T, H, Dv))
    dSf = rng.standard_normal((B, H, Dk, Dv))
    gr = oracle.bwd(q, k, v, g, beta, dO, S0=S0, dS_final=dSf, scale=0.5)
    G = np.exp(np.cumsum(g, axis=1))
    np.testing.assert_array_equal(gr["dv"], 0.0)
    dS0 = 0.5 * np.einsum("bth,bthk,bthv->bhkv", G, q, dO) + G[:, -1][:, :, None, None] * dSf
    np.testing.assert_allclose(gr["dS0"], dS0, rtol=1e-12, atol=1e-13)
    dq = 0.5 * G[..., None] * np.einsum("bhkv,bthv->bthk", S0, dO)
    np.testing.assert_allclose(gr["dq"], dq, rtol=1e-12, atol=1e-13)


def test_page_constants_fixture_is_readable(golden_dir):
    with open(os.path.join(golden_dir, "page_constants.json")) as f:
        c = json.load(f)
    assert c["tolerance_rel_rms_bf16"]["value"] == 0.008
    assert c["tolerance_max_rel_fp32"]["value"] == 3e-4
