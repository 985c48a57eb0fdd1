"""Seeded synthetic inputs for the chunked gated delta rule.

This module draws inputs and nothing else: it holds none of the recurrence's
arithmetic, so both the GPU path's tests/benchmark and the CPU oracle can take
their inputs from it.  Everything is drawn on the host with
``numpy.random.default_rng(seed)`` in float32, in a fixed order
(q_raw, k_raw, v, gate parts, beta_raw, S0, dO), then rounded to the io dtype
with round-to-nearest-even.  The arrays returned are float32 holding values that
are exactly representable in the io dtype, so widening them to float64 (oracle)
or narrowing them to bfloat16 (GPU) is exact.

The five named workloads follow the pages' experiments:

* ``tiny_fp32``   -- Day-1 page ("Research Sprint Day 1", "Experiments"): iid
  Gaussian q/v, L2-normalised Gaussian k; fp32, T=256, d_k=d_v=64.
* ``train_bf16``  -- training shape B=4, T=4096, H=8, d=128 with the gate
  formula of the Day-2 page ("Research Sprint Day 2 - Rooflines", "Building some
  intuition", gates step 5): g = -exp(A_log) * softplus(a + dt_bias).
* ``packed_bf16`` -- the fla issue #1550 workload ("Reproduction and evidence"):
  one packed row of 10240 tokens, sequence lengths [5120, 5120], H=12, K=V=128,
  bounded gates g in [-5, 0), correlated ("asymmetric") q/k, random initial state.
* ``long_bf16``   -- the cuLA issue #126 synthetic case ("Minimal public
  reproduction"): T=65536, H=1, d=128, slow constant decay.
* ``fwdbwd_bf16`` -- Day-2 training shape B=32, T=1024, H=16, d_k=64, d_v=128
  (value expansion 2), forward plus backward with upstream dO.
* ``kda_bf16``    -- the training shape of ``train_bf16`` with one log-decay per
  (token, head, key channel), the gate layout of the cuLA issue #126 page
  ("Minimal public reproduction": g shaped like q, dt_bias per head and
  channel); the values follow the Day-2 gate formula channel by channel.
* ``kda_long_bf16`` -- the cuLA issue #126 synthetic case in its own gate layout:
  T=65536, H=1, d=128, per-channel log-decays uniform in [-1e-3, -1e-4) (slow
  decay), for the segment split.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np


def round_bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32)
    # add 0x7FFF plus the lowest kept bit, then clear the 16 dropped bits; the
    # sum cannot wrap for finite inputs (it carries into the exponent at most)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32).reshape(x.shape)


def _normalize(x: np.ndarray) -> np.ndarray:
    # L2 normalisation over the last axis, in float32 (the operator contract the
    # fla issue #1550 page insists on: normalise in FP32, then cast).
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-30))).astype(np.float32)


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _softplus(x):
    return np.logaddexp(np.float32(0.0), x).astype(np.float32)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    Dk: int
    Dv: int
    io: str = "bf16"                    # "bf16" or "fp32"
    qk: str = "iid"                     # "iid" (q ~ N, k normalised) / "norm_both" / "correlated"
    gate: str = "gdn"                   # "softplus01" / "gdn" / "bounded5" / "const" /
                                        # "gdn_channel" (g shaped like q)
    gate_const: float = -1e-3
    cu_seqlens: Optional[Sequence[int]] = None   # packed row (B must be 1)
    s0_std: Optional[float] = None      # None: no initial state; 0.0: explicit zeros
    with_dO: bool = False
    scale: float = 1.0
    seed: int = 0

    @property
    def num_seqs(self) -> int:
        return len(self.cu_seqlens) - 1 if self.cu_seqlens is not None else self.B

    @property
    def token_heads(self) -> int:
        return self.B * self.T * self.H

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 256, 1, 64, 64, io="fp32", qk="iid",
                          gate="softplus01", seed=0),
    "train_bf16": Workload("train_bf16", 4, 4096, 8, 128, 128, io="bf16", qk="norm_both",
                           gate="gdn", seed=1),
    "packed_bf16": Workload("packed_bf16", 1, 10240, 12, 128, 128, io="bf16",
                            qk="correlated", gate="bounded5", cu_seqlens=(0, 5120, 10240),
                            s0_std=0.1, seed=2),
    "long_bf16": Workload("long_bf16", 1, 65536, 1, 128, 128, io="bf16", qk="iid",
                          gate="const", gate_const=-1e-3, seed=3),
    "fwdbwd_bf16": Workload("fwdbwd_bf16", 32, 1024, 16, 64, 128, io="bf16", qk="norm_both",
                            gate="gdn", s0_std=0.0, with_dO=True, seed=4),
    "kda_bf16": Workload("kda_bf16", 4, 4096, 8, 128, 128, io="bf16", qk="norm_both",
                         gate="gdn_channel", seed=5),
    "kda_long_bf16": Workload("kda_long_bf16", 1, 65536, 1, 128, 128, io="bf16", qk="iid",
                              gate="channel_slow", seed=6),
}


def generate(w: Workload) -> dict:
    """Draw one workload.  Returns float32 arrays (io-dtype-exact) and metadata.

    Shapes: q, k (B, T, H, Dk); v, dO (B, T, H, Dv); g, beta (B, T, H) (g is
    (B, T, H, Dk) for the per-channel gate);
    S0 (N, H, Dk, Dv) or None; cu_seqlens int32 (N+1,) or None.
    """
    if w.cu_seqlens is not None:
        cu = np.asarray(w.cu_seqlens, dtype=np.int32)
        if w.B != 1 or cu[0] != 0 or cu[-1] != w.T or np.any(np.diff(cu) < 0):
            raise ValueError("packed workloads need B == 1 and cu_seqlens 0 .. T, non-decreasing")
    else:
        cu = None
    rng = np.random.default_rng(w.seed)
    B, T, H, Dk, Dv = w.B, w.T, w.H, w.Dk, w.Dv
    cast = round_bf16 if w.io == "bf16" else (lambda a: np.asarray(a, dtype=np.float32))

    def randn(*shape):
        return rng.standard_normal(shape, dtype=np.float32)

    q_raw = randn(B, T, H, Dk)
    k_raw = randn(B, T, H, Dk)
    if w.qk == "iid":
        q = q_raw
        k = _normalize(k_raw)
    elif w.qk == "norm_both":
        q = _normalize(q_raw)
        k = _normalize(k_raw)
    elif w.qk == "correlated":
        # q = normalize(0.8 k_raw + 0.6 noise); the fresh draw q_raw is the noise.
        q = _normalize((np.float32(0.8) * k_raw + np.float32(0.6) * q_raw).astype(np.float32))
        k = _normalize(k_raw)
    else:
        raise ValueError(w.qk)
    v = randn(B, T, H, Dv)

    if w.gate == "softplus01":
        g = (np.float32(-0.1) * _softplus(randn(B, T, H))).astype(np.float32)
    elif w.gate == "gdn":
        a = randn(B, T, H)
        A_log = rng.uniform(0.0, 1.5, size=(H,)).astype(np.float32)
        dt_bias = (np.float32(0.5) * randn(H)).astype(np.float32)
        g = (-np.exp(A_log) * _softplus(a + dt_bias)).astype(np.float32)
    elif w.gate == "bounded5":
        g = (np.float32(-5.0) * _sigmoid(randn(B, T, H))).astype(np.float32)
    elif w.gate == "const":
        g = np.full((B, T, H), w.gate_const, dtype=np.float32)
    elif w.gate == "channel_slow":
        # slow per-channel decay: log-decay per (token, head, key channel) uniform in
        # [-1e-3, -1e-4), so the state forgets over thousands of tokens
        g = (-(1e-4 + 9e-4 * rng.random((B, T, H, Dk)))).astype(np.float32)
    elif w.gate == "gdn_channel":
        a = randn(B, T, H, Dk)
        A_log = rng.uniform(0.0, 1.5, size=(H,)).astype(np.float32)
        dt_bias = (np.float32(0.5) * randn(H, Dk)).astype(np.float32)
        g = (-np.exp(A_log)[:, None] * _softplus(a + dt_bias)).astype(np.float32)
    else:
        raise ValueError(w.gate)
    beta = _sigmoid(randn(B, T, H))

    N = w.num_seqs
    if w.s0_std is None:
        S0 = None
    elif w.s0_std == 0.0:
        S0 = np.zeros((N, H, Dk, Dv), dtype=np.float32)
    else:
        S0 = (np.float32(w.s0_std) * randn(N, H, Dk, Dv)).astype(np.float32)
    dO = cast(randn(B, T, H, Dv)) if w.with_dO else None

    return {
        "q": cast(q), "k": cast(k), "v": cast(v),
        "g": g.astype(np.float32), "beta": beta.astype(np.float32),
        "S0": S0, "dO": dO, "cu_seqlens": cu,
        "scale": float(w.scale), "io": w.io, "workload": w,
    }
