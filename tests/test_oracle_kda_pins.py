"""Pins of the per-key-channel-decay oracle (``oracle.kda_fwd``) to facts other
than itself (CPU only).

* equal decays on every channel reduce it to the scalar-gate recurrence, whose
  C oracle is pinned in tests/test_oracle_pins.py;
* explicit d_k x d_k transition matrices M_t = (I - beta_t k_t k_t^T) diag(a_t),
  stepped and unrolled, on tiny inputs;
* closed forms: beta = 0 (pure per-channel decay of S0), a = 0 on every channel
  with beta = 1 and unit keys (the state is the last outer product), and keys
  confined to a channel subset (the other rows only decay);
* packed sequences equal separate dense calls.

A decay applied to the value axis instead of the key axis, a dropped forget, the
output read before the write, or a sign error fails at least one of them.  The
last test checks the chunk algebra the GPU kernels evaluate against the oracle.
"""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(2024)


def _inputs(B, T, H, Dk, Dv, rng, gscale=0.3, S0=True):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    g = -gscale * rng.random((B, T, H, Dk))
    beta = rng.random((B, T, H))
    s0 = rng.standard_normal((B, H, Dk, Dv)) if S0 else None
    return q, k, v, g, beta, s0


def test_equal_channel_decays_reduce_to_scalar_gate():
    q, k, v, g, beta, S0 = _inputs(2, 37, 3, 8, 5, RNG)
    gs = g[..., 0]
    o, Sf = oracle.kda_fwd(q, k, v, np.repeat(gs[..., None], 8, axis=-1), beta, S0=S0, scale=0.7)
    o_ref, Sf_ref = oracle.fwd(q, k, v, gs, beta, S0=S0, scale=0.7, nthreads=1)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Sf, Sf_ref, rtol=0, atol=1e-13)


def test_transition_matrices_brute_force():
    T, Dk, Dv = 9, 4, 3
    q, k, v, g, beta, S0 = _inputs(1, T, 1, Dk, Dv, RNG, gscale=0.8)
    beta *= 1.9  # the (0, 2) range of negative eigenvalues
    o, Sf = oracle.kda_fwd(q, k, v, g, beta, S0=S0, scale=1.3)
    S = S0[0, 0].copy()
    Ms, Bs = [], []
    for t in range(T):
        kt, bt = k[0, t, 0], beta[0, t, 0]
        M = (np.eye(Dk) - bt * np.outer(kt, kt)) @ np.diag(np.exp(g[0, t, 0]))
        Bt = bt * np.outer(kt, v[0, t, 0])
        S = M @ S + Bt
        Ms.append(M)
        Bs.append(Bt)
        np.testing.assert_allclose(o[0, t, 0], 1.3 * S.T @ q[0, t, 0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(Sf[0, 0], S, rtol=0, atol=1e-13)
    # unrolled: S_T = Phi(T, 0) S0 + sum_t Phi(T, t) B_t,  Phi(T, t) = M_T ... M_{t+1}
    acc = np.zeros((Dk, Dv))
    phi = np.eye(Dk)
    for t in reversed(range(T)):
        acc += phi @ Bs[t]
        phi = phi @ Ms[t]
    np.testing.assert_allclose(Sf[0, 0], phi @ S0[0, 0] + acc, rtol=0, atol=1e-13)


def test_zero_beta_is_pure_channel_decay():
    q, k, v, g, beta, S0 = _inputs(1, 20, 2, 6, 4, RNG)
    beta[:] = 0.0
    o, Sf = oracle.kda_fwd(q, k, v, g, beta, S0=S0, scale=0.5)
    cum = np.cumsum(g[0], axis=0)                      # (T, H, Dk)
    np.testing.assert_allclose(Sf[0], np.exp(cum[-1])[:, :, None] * S0[0], rtol=1e-14, atol=0)
    for t in range(20):
        St = np.exp(cum[t])[:, :, None] * S0[0]
        np.testing.assert_allclose(o[0, t], 0.5 * np.einsum("hkv,hk->hv", St, q[0, t]), rtol=0, atol=1e-14)


def test_full_forget_keeps_only_the_last_write():
    q, k, v, g, beta, S0 = _inputs(1, 12, 2, 5, 3, RNG)
    g[:] = -np.inf
    beta[:] = 1.0
    o, Sf = oracle.kda_fwd(q, k, v, g, beta, S0=S0, scale=1.0)
    qk = np.sum(q[0] * k[0], axis=-1)                 # (T, H)
    np.testing.assert_allclose(o[0], qk[:, :, None] * v[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(Sf[0], k[0, -1][:, :, None] * v[0, -1][:, None, :], rtol=0, atol=1e-14)


def test_keys_on_a_channel_subset():
    # keys live on channels 0..2 only: rows 3.. of the state only decay, rows 0..2
    # follow the same recurrence restricted to those channels
    q, k, v, g, beta, S0 = _inputs(1, 15, 1, 6, 4, RNG)
    k[..., 3:] = 0.0
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    _, Sf = oracle.kda_fwd(q, k, v, g, beta, S0=S0)
    cum = np.sum(g[0, :, 0], axis=0)
    np.testing.assert_allclose(Sf[0, 0, 3:], np.exp(cum[3:])[:, None] * S0[0, 0, 3:], rtol=1e-14, atol=0)
    _, Sf_sub = oracle.kda_fwd(q[..., :3], k[..., :3], v, g[..., :3], beta, S0=S0[:, :, :3])
    np.testing.assert_allclose(Sf[0, 0, :3], Sf_sub[0, 0], rtol=0, atol=1e-14)


def test_packed_equals_dense_sequences():
    lens = [7, 0, 19]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta, _ = _inputs(1, cu[-1], 2, 4, 3, RNG)
    S0 = RNG.standard_normal((3, 2, 4, 3))
    o, Sf = oracle.kda_fwd(q, k, v, g, beta, cu_seqlens=cu, S0=S0, scale=0.9)
    for n in range(3):
        sl = slice(cu[n], cu[n + 1])
        o_n, Sf_n = oracle.kda_fwd(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], S0=S0[n:n + 1],
                                   scale=0.9)
        np.testing.assert_allclose(o[sl], o_n[0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(Sf[n], Sf_n[0], rtol=0, atol=1e-14)


def _chunk_model(q, k, v, g, beta, S0, scale, C):
    """The chunk algebra of the GPU kernels, in float64 (one dense sequence, one
    head): gamma = cumsum(g) per channel inside the chunk;
    A_ij = beta_i sum_c k_ic k_jc exp(gamma_ic - gamma_jc) (j < i);
    P_ij = sum_c q_ic k_jc exp(gamma_ic - gamma_jc) (j <= i);
    E = (I + A)^-1 diag(beta) (V - (K o Gamma) S);  O = scale ((Q o Gamma) S + P E);
    S <- diag(Gamma_n) S + (K o exp(gamma_n - gamma))^T E."""
    T = q.shape[0]
    S = S0.copy()
    o = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, C):
        sl = slice(c0, min(c0 + C, T))
        Q, K, V, G, b = q[sl], k[sl], v[sl], np.cumsum(g[sl], axis=0), beta[sl]
        n = Q.shape[0]
        D = np.exp(G[:, None, :] - G[None, :, :])        # (i, j, c), used for j <= i only
        A = np.tril(b[:, None] * np.einsum("ic,jc,ijc->ij", K, K, D), -1)
        P = np.tril(np.einsum("ic,jc,ijc->ij", Q, K, D))
        Tm = np.linalg.inv(np.eye(n) + A)
        E = Tm @ (b[:, None] * (V - (K * np.exp(G)) @ S))
        o[sl] = scale * ((Q * np.exp(G)) @ S + P @ E)
        S = np.exp(G[-1])[:, None] * S + (K * np.exp(G[-1][None, :] - G)).T @ E
    return o, S


@pytest.mark.parametrize("C", [64, 16])
def test_chunk_algebra_matches_oracle(C):
    T = 150  # two full chunks of 64 and a ragged tail of 22
    q, k, v, g, beta, S0 = _inputs(1, T, 1, 8, 6, RNG, gscale=2.0)
    o, Sf = oracle.kda_fwd(q, k, v, g, beta, S0=S0, scale=0.6)
    o_c, S_c = _chunk_model(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0], S0[0, 0], 0.6, C)
    np.testing.assert_allclose(o_c, o[0, :, 0], rtol=0, atol=1e-12 * np.abs(o).max())
    np.testing.assert_allclose(S_c, Sf[0, 0], rtol=0, atol=1e-12 * np.abs(Sf).max())
