"""CPU fp64 oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the package smoke check (``__graft_entry__.smoke``) and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library never
imports, links or calls it, and it shares no code with the GPU path.

``prologue`` / ``epilogue`` are the input prologue and the output epilogue in
float64 numpy (the normalisation and the
gate formulas written out; pinned in tests/test_oracle_pins.py).

``kda_fwd`` is the same recurrence with one decay per key channel (numpy,
float64) and ``kda_bwd`` its reverse mode (pinned in tests/test_oracle_kda_pins.py
and tests/test_oracle_kda_bwd_pins.py).

``fwd`` / ``bwd`` wrap ``liboracle.so`` (built from ``gdn_oracle.c`` with gcc):
the plain token-by-token recurrence of the Day-1 page ("Research Sprint Day 1",
section "The GDN update": forget, read, write the error, read with the query),
in double precision, and its reverse mode.  Every input is widened to float64
exactly as given (bf16 and fp32 values are exactly representable).

Array conventions (numpy):
  dense  : q, k (B, T, H, Dk); v (B, T, H, Dv); g, beta (B, T, H); cu_seqlens None
  packed : q, k (Ttot, H, Dk); v (Ttot, H, Dv); g, beta (Ttot, H); cu_seqlens (N+1,)
  S0, S_final, dS_final, dS0 : (N, H, Dk, Dv), N = B for dense inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

# x86-64-v3 (AVX2 + FMA) rather than -march=native: the library is built on one
# host and may run on another.
GCC_CMD = ["gcc", "-O3", "-march=x86-64-v3", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", "-Wno-unused-parameter", "-pthread",
           _SRC, "-o", _LIB, "-lm"]


def build() -> str:
    """Compile liboracle.so in place (always recompiles)."""
    tmp = _LIB + ".tmp"
    cmd = list(GCC_CMD)
    cmd[cmd.index(_LIB)] = tmp
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    lib.oracle_fwd.argtypes = [I, P, I, I, I, P, P, P, P, P, P, D, P, P, I]
    lib.oracle_fwd.restype = I
    lib.oracle_bwd.argtypes = [I, P, I, I, I, P, P, P, P, P, P, D, P, P, P, P, P, P, P, P, I]
    lib.oracle_bwd.restype = I
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _f64(x):
    return None if x is None else np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _pack(q, k, v, g, beta, cu_seqlens):
    """Bring dense (B,T,...) inputs to the packed layout with uniform cu_seqlens."""
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    if cu_seqlens is None:
        if q.ndim != 4:
            raise ValueError("dense inputs must be (B, T, H, D)")
        B, T, H, _ = q.shape
        cu = np.arange(B + 1, dtype=np.int64) * T
        shape = (B, T)
        q, k, v = (x.reshape(B * T, H, x.shape[-1]) for x in (q, k, v))
        g, beta = (x.reshape(B * T, H) for x in (g, beta))
    else:
        if q.ndim == 4 and q.shape[0] == 1:  # (1, Ttot, H, D): one packed row
            q, k, v = (x[0] for x in (q, k, v))
            g, beta = (x.reshape(x.shape[-2:]) for x in (g, beta))
        if q.ndim != 3:
            raise ValueError("packed inputs must be (Ttot, H, D) or (1, Ttot, H, D)")
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        shape = (q.shape[0],)
        if cu[0] != 0 or cu[-1] != q.shape[0] or np.any(np.diff(cu) < 0):
            raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at Ttot")
    return q, k, v, g, beta, cu, shape


def fwd(q, k, v, g, beta, cu_seqlens=None, S0=None, scale=1.0, nthreads=None):
    """Return (o, S_final) in float64; o has v's leading shape."""
    lib = _load()
    q, k, v, g, beta, cu, shape = _pack(q, k, v, g, beta, cu_seqlens)
    N = len(cu) - 1
    H, Dk = q.shape[1], q.shape[2]
    Dv = v.shape[2]
    S0 = _f64(S0)
    if S0 is not None and S0.shape != (N, H, Dk, Dv):
        raise ValueError(f"S0 must be {(N, H, Dk, Dv)}")
    o = np.zeros((q.shape[0], H, Dv))
    Sf = np.zeros((N, H, Dk, Dv))
    rc = lib.oracle_fwd(N, _ptr(cu), H, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                        _ptr(beta), _ptr(S0), float(scale), _ptr(o), _ptr(Sf),
                        int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_fwd failed with code {rc}")
    return o.reshape(shape + (H, Dv)), Sf


def bwd(q, k, v, g, beta, dO, cu_seqlens=None, S0=None, dS_final=None, scale=1.0,
        nthreads=None):
    """Return dict dq, dk, dv, dg, dbeta, dS0 (float64) of L = <o, dO> + <S_final, dS_final>."""
    lib = _load()
    q, k, v, g, beta, cu, shape = _pack(q, k, v, g, beta, cu_seqlens)
    N = len(cu) - 1
    H, Dk = q.shape[1], q.shape[2]
    Dv = v.shape[2]
    dO = _f64(dO).reshape(q.shape[0], H, Dv)
    S0 = _f64(S0)
    dSf = _f64(dS_final)
    out = {
        "dq": np.zeros((q.shape[0], H, Dk)),
        "dk": np.zeros((q.shape[0], H, Dk)),
        "dv": np.zeros((q.shape[0], H, Dv)),
        "dg": np.zeros((q.shape[0], H)),
        "dbeta": np.zeros((q.shape[0], H)),
        "dS0": np.zeros((N, H, Dk, Dv)),
    }
    rc = lib.oracle_bwd(N, _ptr(cu), H, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                        _ptr(beta), _ptr(S0), float(scale), _ptr(dO), _ptr(dSf),
                        _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                        _ptr(out["dbeta"]), _ptr(out["dS0"]),
                        int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_bwd failed with code {rc}")
    for name in ("dq", "dk", "dv"):
        out[name] = out[name].reshape(shape + out[name].shape[1:])
    for name in ("dg", "dbeta"):
        out[name] = out[name].reshape(shape + (H,))
    return out


def prologue(q_raw, k_raw, a, b, A_log=None, dt_bias=None, gate="gdn", allow_neg_eigval=False):
    """The operator's inputs from the raw projections, in float64.

    q = q_raw / ||q_raw||, k = k_raw / ||k_raw|| (L2 over the last axis; the
    normalisation the fla issue #1550 page, "Proposed scope", places before the
    cast); beta = sigmoid(b), doubled when negative eigenvalues are allowed (range
    (0, 2), "Research Sprint Day 2", "Building some intuition", gates); and the
    log-decay g = -exp(A_log[h]) softplus(a + dt_bias[h]) (the same page's gate
    formula) or, for gate == "bounded5", g = -5 sigmoid(a); for gate ==
    "gdn_channel" the first form channel by channel, a shaped like q and dt_bias
    (H, Dk) (the KDA gate layout of the cuLA issue #126 page, "Minimal public
    reproduction").  Returns float64 arrays (q, k, g, beta) of the input shapes.
    """
    q = _f64(q_raw)
    k = _f64(k_raw)
    qn = np.sqrt(np.sum(q * q, axis=-1, keepdims=True))
    kn = np.sqrt(np.sum(k * k, axis=-1, keepdims=True))
    q = q / np.maximum(qn, 1e-30)
    k = k / np.maximum(kn, 1e-30)
    a = _f64(a)
    b = _f64(b)
    sig_b = 1.0 / (1.0 + np.exp(-b))
    beta = 2.0 * sig_b if allow_neg_eigval else sig_b
    if gate == "gdn":
        x = a + _f64(dt_bias)
        softplus = np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))
        g = -np.exp(_f64(A_log)) * softplus
    elif gate == "gdn_channel":
        x = a + _f64(dt_bias)                          # (..., H, Dk) + (H, Dk)
        softplus = np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))
        g = -np.exp(_f64(A_log))[:, None] * softplus
    elif gate == "bounded5":
        g = -5.0 / (1.0 + np.exp(-a))
    else:
        raise ValueError(gate)
    return q, k, g, beta


def epilogue(o, z, weight=None, eps=1e-6):
    """The gated, normalised output in float64: per (token, head) over the last
    axis, y = o / sqrt(mean(o^2) + eps) * weight * silu(z) with silu(z) =
    z / (1 + exp(-z)) ("Research Sprint Day 2", "Building some intuition", step 7:
    normalise per head, then gate).  weight None means ones."""
    o = _f64(o)
    z = _f64(z)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    w = 1.0 if weight is None else _f64(weight)
    return o / rms * w * (z / (1.0 + np.exp(-z)))


def _kda_unpack(q, k, v, g, beta, cu_seqlens):
    """Float64 copies flattened to (Ttot, H, .) rows, the sequence offsets and the
    leading shape of the outputs (dense (B, T) or packed (Ttot,))."""
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    if g.shape != q.shape:
        raise ValueError("g must be shaped like q (one log-decay per key channel)")
    if cu_seqlens is None:
        if q.ndim != 4:
            raise ValueError("dense inputs must be (B, T, H, D)")
        B, T = q.shape[:2]
        cu = np.arange(B + 1, dtype=np.int64) * T
        lead = (B, T)
    else:
        if q.ndim == 4 and q.shape[0] == 1:
            q, k, v, g, beta = q[0], k[0], v[0], g[0], beta.reshape(beta.shape[-2:])
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        lead = (q.shape[0],)
        if cu[0] != 0 or cu[-1] != q.shape[0] or np.any(np.diff(cu) < 0):
            raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at Ttot")
    H, Dk = q.shape[-2:]
    Dv = v.shape[-1]
    q, k, g = (x.reshape(-1, H, Dk) for x in (q, k, g))
    return q, k, v.reshape(-1, H, Dv), g, beta.reshape(-1, H), cu, lead


def kda_fwd(q, k, v, g, beta, cu_seqlens=None, S0=None, scale=1.0):
    """Gated delta rule with a per-key-channel decay, token by token, in float64.

    The update of "Research Sprint Day 1" ("The GDN update") with the scalar
    forget factor replaced by a diagonal one: g holds one log-decay per (token,
    head, key channel), the gate layout of the cuLA issue #126 page ("Minimal
    public reproduction", g shaped like q).  Per token, with a = exp(g_t) of
    length Dk:
        S <- diag(a) S,  r = S^T k_t,  e = beta_t (v_t - r),  S <- S + k_t e^T,
        o_t = scale S^T q_t.
    Shapes: q, k, g (B, T, H, Dk) or packed (Ttot, H, Dk); v (..., H, Dv);
    beta (..., H); S0 / S_final (N, H, Dk, Dv).  Returns (o, S_final) in float64.
    """
    q, k, v, g, beta, cu, lead = _kda_unpack(q, k, v, g, beta, cu_seqlens)
    H, Dk = q.shape[-2:]
    Dv = v.shape[-1]
    N = len(cu) - 1
    S0 = _f64(S0)
    if S0 is not None and S0.shape != (N, H, Dk, Dv):
        raise ValueError(f"S0 must be {(N, H, Dk, Dv)}")
    o = np.zeros((q.shape[0], H, Dv))
    Sf = np.zeros((N, H, Dk, Dv))
    for n in range(N):
        S = np.zeros((H, Dk, Dv)) if S0 is None else S0[n].copy()
        for t in range(cu[n], cu[n + 1]):
            S *= np.exp(g[t])[:, :, None]                        # forget, per key channel
            r = np.einsum("hkv,hk->hv", S, k[t])                 # read the old value
            e = beta[t][:, None] * (v[t] - r)                    # written error
            S += k[t][:, :, None] * e[:, None, :]                # write
            o[t] = scale * np.einsum("hkv,hk->hv", S, q[t])      # read after the write
        Sf[n] = S
    return o.reshape(lead + (H, Dv)), Sf


def kda_bwd(q, k, v, g, beta, dO, cu_seqlens=None, S0=None, dS_final=None, scale=1.0):
    """Reverse mode of ``kda_fwd``, token by token, in float64.

    Gradients of L = <o, dO> + <S_final, dS_final> with respect to q, k, v, the
    per-channel log-decays g, beta and S0.  The forward states S_0 .. S_L of each
    sequence are kept, then the steps of ``kda_fwd`` are undone last to first
    (the same forget / read / write / read order of "Research Sprint Day 1",
    "The GDN update", with the forget factor diagonal over key channels):
        o_t = scale S_t^T q_t     ->  dS += scale q_t do_t^T,  dq_t = scale S_t do_t
        S_t = S' + k_t e^T        ->  dk_t = dS e,  de = dS^T k_t
        e = beta_t (v_t - r)      ->  dv_t = beta_t de,  dbeta_t = <de, v_t - r>,
                                      dr = -beta_t de
        r = S'^T k_t              ->  dS' = dS + k_t dr^T,  dk_t += S' dr
        S' = diag(a) S_{t-1}      ->  dg_t = a o rowsum(dS' o S_{t-1}),
                                      dS_{t-1} = diag(a) dS'
    with a = exp(g_t).  Shapes as ``kda_fwd``; dg has g's shape.  Returns a dict
    dq, dk, dv, dg, dbeta, dS0.
    """
    q, k, v, g, beta, cu, lead = _kda_unpack(q, k, v, g, beta, cu_seqlens)
    H, Dk = q.shape[-2:]
    Dv = v.shape[-1]
    N = len(cu) - 1
    dO = _f64(dO).reshape(-1, H, Dv)
    S0 = _f64(S0)
    dSf = _f64(dS_final)
    for name, x in (("S0", S0), ("dS_final", dSf)):
        if x is not None and x.shape != (N, H, Dk, Dv):
            raise ValueError(f"{name} must be {(N, H, Dk, Dv)}")
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v),
           "dg": np.zeros_like(g), "dbeta": np.zeros_like(beta), "dS0": np.zeros((N, H, Dk, Dv))}
    for n in range(N):
        t0, t1 = cu[n], cu[n + 1]
        S = np.zeros((H, Dk, Dv)) if S0 is None else S0[n].copy()
        states = [S.copy()]
        for t in range(t0, t1):
            S *= np.exp(g[t])[:, :, None]
            r = np.einsum("hkv,hk->hv", S, k[t])
            S += k[t][:, :, None] * (beta[t][:, None] * (v[t] - r))[:, None, :]
            states.append(S.copy())
        dS = np.zeros((H, Dk, Dv)) if dSf is None else dSf[n].copy()
        for t in range(t1 - 1, t0 - 1, -1):
            a = np.exp(g[t])
            Sprev = states[t - t0]
            Sp = a[:, :, None] * Sprev                                   # S'
            r = np.einsum("hkv,hk->hv", Sp, k[t])
            e = beta[t][:, None] * (v[t] - r)
            Scur = states[t - t0 + 1]
            dS += scale * q[t][:, :, None] * dO[t][:, None, :]
            out["dq"][t] = scale * np.einsum("hkv,hv->hk", Scur, dO[t])
            dk = np.einsum("hkv,hv->hk", dS, e)
            de = np.einsum("hkv,hk->hv", dS, k[t])
            out["dv"][t] = beta[t][:, None] * de
            out["dbeta"][t] = np.einsum("hv,hv->h", de, v[t] - r)
            dr = -beta[t][:, None] * de
            dS += k[t][:, :, None] * dr[:, None, :]
            out["dk"][t] = dk + np.einsum("hkv,hv->hk", Sp, dr)
            out["dg"][t] = a * np.einsum("hkv,hkv->hk", dS, Sprev)
            dS *= a[:, :, None]
        out["dS0"][n] = dS
    for name in ("dq", "dk", "dv", "dg"):
        out[name] = out[name].reshape(lead + out[name].shape[1:])
    out["dbeta"] = out["dbeta"].reshape(lead + (H,))
    return out
