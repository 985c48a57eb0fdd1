"""Pins of the per-key-channel-decay reverse mode (``oracle.kda_bwd``) to facts
other than itself (CPU only).

* central finite differences of the forward (``oracle.kda_fwd``, itself pinned in
  tests/test_oracle_kda_pins.py) on tiny inputs, for every input the loss
  L = <o, dO> + <S_final, dS_final> depends on, element by element;
* equal decays on every channel reduce it to the scalar-gate reverse mode of the
  C oracle (pinned in tests/test_oracle_pins.py): the same dq, dk, dv, dbeta and
  dS0, and the per-channel dg summed over channels is the scalar dg;
* packed sequences equal separate dense calls.

A dropped term of any reverse step (the read's dS' += k dr^T, the write's dk),
a decay gradient taken against S' instead of S_{t-1}, or a transposed operand
fails the finite differences.
"""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(77)


def _inputs(B, T, H, Dk, Dv, rng, gscale=0.5):
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    g = -gscale * rng.random((B, T, H, Dk))
    beta = rng.random((B, T, H))
    S0 = rng.standard_normal((B, H, Dk, Dv))
    dO = rng.standard_normal((B, T, H, Dv))
    dSf = rng.standard_normal((B, H, Dk, Dv))
    return dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0), dO, dSf


def _loss(x, dO, dSf, scale):
    o, Sf = oracle.kda_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], S0=x["S0"], scale=scale)
    return float(np.sum(o * dO) + np.sum(Sf * dSf))


def test_finite_differences_every_input():
    scale = 0.8
    x, dO, dSf = _inputs(2, 6, 2, 4, 3, RNG)
    x["beta"] = x["beta"] * 1.9  # the (0, 2) range
    grads = oracle.kda_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], dO, S0=x["S0"], dS_final=dSf,
                           scale=scale)
    name_of = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "S0": "dS0"}
    h = 1e-6
    for key, gname in name_of.items():
        fd = np.zeros_like(x[key])
        for idx in np.ndindex(x[key].shape):
            orig = x[key][idx]
            x[key][idx] = orig + h
            lp = _loss(x, dO, dSf, scale)
            x[key][idx] = orig - h
            lm = _loss(x, dO, dSf, scale)
            x[key][idx] = orig
            fd[idx] = (lp - lm) / (2 * h)
        got = grads[gname]
        assert got.shape == fd.shape, gname
        err = np.max(np.abs(got - fd)) / max(1.0, np.max(np.abs(fd)))
        assert err < 1e-7, (gname, err)


def test_equal_channel_decays_reduce_to_scalar_gate():
    x, dO, dSf = _inputs(2, 21, 3, 8, 5, RNG)
    gs = x["g"][..., 0]
    gk = np.repeat(gs[..., None], 8, axis=-1)
    got = oracle.kda_bwd(x["q"], x["k"], x["v"], gk, x["beta"], dO, S0=x["S0"], dS_final=dSf, scale=0.6)
    ref = oracle.bwd(x["q"], x["k"], x["v"], gs, x["beta"], dO, S0=x["S0"], dS_final=dSf, scale=0.6,
                     nthreads=1)
    for name in ("dq", "dk", "dv", "dbeta", "dS0"):
        np.testing.assert_allclose(got[name], ref[name], rtol=0, atol=1e-12, err_msg=name)
    np.testing.assert_allclose(got["dg"].sum(-1), ref["dg"], rtol=0, atol=1e-12)


def test_packed_equals_dense_sequences():
    x, dO, dSf = _inputs(3, 11, 2, 4, 6, RNG)
    lens = [11, 4, 7]
    cu = np.concatenate([[0], np.cumsum(lens)])
    pk = {key: np.concatenate([x[key][b, :lens[b]] for b in range(3)]) for key in ("q", "k", "v", "g", "beta")}
    dOp = np.concatenate([dO[b, :lens[b]] for b in range(3)])
    got = oracle.kda_bwd(pk["q"], pk["k"], pk["v"], pk["g"], pk["beta"], dOp, cu_seqlens=cu, S0=x["S0"],
                         dS_final=dSf)
    for b in range(3):
        L = lens[b]
        one = oracle.kda_bwd(x["q"][b:b + 1, :L], x["k"][b:b + 1, :L], x["v"][b:b + 1, :L], x["g"][b:b + 1, :L],
                             x["beta"][b:b + 1, :L], dO[b:b + 1, :L], S0=x["S0"][b:b + 1],
                             dS_final=dSf[b:b + 1])
        sl = slice(cu[b], cu[b + 1])
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            np.testing.assert_allclose(got[name][sl], one[name][0], rtol=0, atol=1e-13, err_msg=name)
        np.testing.assert_allclose(got["dS0"][b], one["dS0"][0], rtol=0, atol=1e-13)


@pytest.mark.parametrize("plant", ["no_read_term", "dg_against_S_prime"])
def test_planted_mistakes_fail_the_finite_differences(plant, monkeypatch):
    """The finite-difference pin is sharp enough to see a one-term mistake."""
    x, dO, dSf = _inputs(1, 4, 1, 3, 2, RNG)
    good = oracle.kda_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], dO, S0=x["S0"], dS_final=dSf)
    # reference gradients of g and k by finite differences
    h = 1e-6
    fd = {}
    for key in ("g", "k"):
        arr = np.zeros_like(x[key])
        for idx in np.ndindex(x[key].shape):
            orig = x[key][idx]
            x[key][idx] = orig + h
            lp = _loss(x, dO, dSf, 1.0)
            x[key][idx] = orig - h
            lm = _loss(x, dO, dSf, 1.0)
            x[key][idx] = orig
            arr[idx] = (lp - lm) / (2 * h)
        fd[key] = arr
    assert np.max(np.abs(good["dg"] - fd["g"])) < 1e-7
    assert np.max(np.abs(good["dk"] - fd["k"])) < 1e-7
    # the planted variants, written out here on the CPU
    q, k, v, g, beta = (x[n][0, :, 0] for n in ("q", "k", "v", "g", "beta"))
    S = x["S0"][0, 0].copy()
    states = [S.copy()]
    for t in range(4):
        S = np.exp(g[t])[:, None] * S
        r = S.T @ k[t]
        S = S + np.outer(k[t], beta[t] * (v[t] - r))
        states.append(S.copy())
    dS = dSf[0, 0].copy()
    dg = np.zeros_like(g)
    dk = np.zeros_like(k)
    for t in range(3, -1, -1):
        a = np.exp(g[t])
        Sp = a[:, None] * states[t]
        r = Sp.T @ k[t]
        e = beta[t] * (v[t] - r)
        dS = dS + np.outer(q[t], dO[0, t, 0])
        dk[t] = dS @ e
        de = dS.T @ k[t]
        dr = -beta[t] * de
        if plant != "no_read_term":
            dS = dS + np.outer(k[t], dr)
        dk[t] += Sp @ dr
        dg[t] = a * np.sum(dS * (Sp if plant == "dg_against_S_prime" else states[t]), axis=1)
        dS = a[:, None] * dS
    bad = max(np.max(np.abs(dg - fd["g"][0, :, 0])), np.max(np.abs(dk - fd["k"][0, :, 0])))
    assert bad > 1e-4, plant


def _chunk_bwd_model(q, k, v, g, beta, S0, dO, dSf, scale, C):
    """The chunk algebra of the GPU backward, in float64 (one sequence, one head).
    Per chunk, with gamma = cumsum(g), Gamma = exp(gamma), Kd = K o Gamma,
    Qd = Q o Gamma, Kb = K o exp(gamma_n - gamma), Ab_ij = sum_c k_ic k_jc
    exp(gamma_ic - gamma_jc) (j < i), A = diag(beta) Ab, T = (I + A)^-1,
    P_ij = sum_c q_ic k_jc exp(gamma_ic - gamma_jc) (j <= i):
      state pass    S_c before every chunk;
      dS pass       dS' (after the chunk), dE = P^T dOs + Kb dS', F = (T diag(beta))^T dE,
                    dS <- diag(Gamma_n) dS' + Qd^T dOs - Kd^T F;
      gradients     R = V - Kd S, E = T diag(beta) R, G = T^T dE, dv = beta o G,
                    dbeta = rowsum(G o R) + rowsum(dA o Ab), dA = -G E^T (j < i),
                    dP = dOs E^T (j <= i), dKd = -F S^T, dQd = dOs S^T, dKb = E dS'^T,
                    and through the decays: for M_ij = sum_c x_ic y_jc D_ijc with
                    D_ijc = exp(gamma_ic - gamma_jc), dx_ic = sum_j dM_ij y_jc D_ijc,
                    dy_jc = sum_i dM_ij x_ic D_ijc and dgamma += x o dx - y o dy (M = P with
                    x = q, y = k; M = Ab with x = y = k, dM = diag(beta) dA); dg is the
                    reverse cumulative sum of dgamma over the chunk plus dgamma_n."""
    T = q.shape[0]
    chunks = [slice(c0, min(c0 + C, T)) for c0 in range(0, T, C)]
    S = S0.copy()
    parts, states = [], []
    for sl in chunks:
        Q, K, V, b = q[sl], k[sl], v[sl], beta[sl]
        G = np.cumsum(g[sl], axis=0)
        n = Q.shape[0]
        D = np.exp(G[:, None, :] - G[None, :, :])
        Ab = np.tril(np.einsum("ic,jc,ijc->ij", K, K, D), -1)
        Pm = np.tril(np.einsum("ic,jc,ijc->ij", Q, K, D))
        Tm = np.linalg.inv(np.eye(n) + b[:, None] * Ab)
        Kd, Qd, Kb = K * np.exp(G), Q * np.exp(G), K * np.exp(G[-1][None, :] - G)
        parts.append(dict(G=G, D=D, Ab=Ab, Pm=Pm, Tm=Tm, Kd=Kd, Qd=Qd, Kb=Kb))
        states.append(S.copy())
        E = Tm @ (b[:, None] * (V - Kd @ S))
        S = np.exp(G[-1])[:, None] * S + Kb.T @ E
    dS = dSf.copy()
    dafter = [None] * len(chunks)
    for ci in range(len(chunks) - 1, -1, -1):
        sl, pt = chunks[ci], parts[ci]
        dafter[ci] = dS.copy()
        dOs = scale * dO[sl]
        dE = pt["Pm"].T @ dOs + pt["Kb"] @ dS
        F = (pt["Tm"] * beta[sl][None, :]).T @ dE
        dS = np.exp(pt["G"][-1])[:, None] * dS + pt["Qd"].T @ dOs - pt["Kd"].T @ F
    out = {"dS0": dS, "dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v),
           "dg": np.zeros_like(g), "dbeta": np.zeros_like(beta)}
    for ci, sl in enumerate(chunks):
        pt, S, dSa = parts[ci], states[ci], dafter[ci]
        Q, K, V, b, D = q[sl], k[sl], v[sl], beta[sl], pt["D"]
        dOs = scale * dO[sl]
        R = V - pt["Kd"] @ S
        E = pt["Tm"] @ (b[:, None] * R)
        dE = pt["Pm"].T @ dOs + pt["Kb"] @ dSa
        Gm = pt["Tm"].T @ dE
        F = b[:, None] * Gm
        dA = np.tril(-Gm @ E.T, -1)
        dbeta = np.sum(Gm * R, axis=1) + np.sum(dA * pt["Ab"], axis=1)
        dAb = b[:, None] * dA
        dP = np.tril(dOs @ E.T)
        dKd, dQd, dKb = -F @ S.T, dOs @ S.T, E @ dSa.T
        Gam, eb = np.exp(pt["G"]), np.exp(pt["G"][-1][None, :] - pt["G"])
        # pair products through the per-channel decays (D_ijc = exp(gamma_ic - gamma_jc))
        dq_P = np.einsum("ij,jc,ijc->ic", dP, K, D)
        dk_P = np.einsum("ij,ic,ijc->jc", dP, Q, D)
        dk_A1 = np.einsum("ij,jc,ijc->ic", dAb, K, D)
        dk_A2 = np.einsum("ij,ic,ijc->jc", dAb, K, D)
        dq = dQd * Gam + dq_P
        dk = dKd * Gam + dKb * eb + dk_P + dk_A1 + dk_A2
        dgam = dKd * K * Gam + dQd * Q * Gam - dKb * K * eb + Q * dq_P - K * dk_P + K * dk_A1 - K * dk_A2
        dgam_n = np.sum(dKb * K * eb, axis=0) + np.exp(pt["G"][-1]) * np.sum(dSa * S, axis=1)
        dg = np.cumsum(dgam[::-1], axis=0)[::-1] + dgam_n[None, :]
        out["dq"][sl], out["dk"][sl], out["dv"][sl] = dq, dk, F
        out["dg"][sl], out["dbeta"][sl] = dg, dbeta
    return out


@pytest.mark.parametrize("C", [64, 16])
def test_chunk_backward_algebra_matches_oracle(C):
    T = 150  # two full chunks of 64 and a ragged tail of 22
    x, dO, dSf = _inputs(1, T, 1, 8, 6, RNG, gscale=2.0)
    x["beta"] = x["beta"] * 1.9
    ref = oracle.kda_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], dO, S0=x["S0"], dS_final=dSf, scale=0.6)
    got = _chunk_bwd_model(*(x[n][0, :, 0] for n in ("q", "k", "v", "g", "beta")), x["S0"][0, 0],
                           dO[0, :, 0], dSf[0, 0], 0.6, C)
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        r = ref[name][0, :, 0]
        np.testing.assert_allclose(got[name], r, rtol=0, atol=1e-10 * np.abs(r).max(), err_msg=name)
    np.testing.assert_allclose(got["dS0"], ref["dS0"][0, 0], rtol=0, atol=1e-10 * np.abs(ref["dS0"]).max())
