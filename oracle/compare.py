"""Error metrics used to compare a result with the oracle -- TEST INFRASTRUCTURE.

All are computed in float64 over a whole tensor (or a slice the caller picks).

* ``max_rel(x, ref) = max|x - ref| / max|ref|`` -- the "max relative error
  across all elements" of the Day-1 page ("Research Sprint Day 1", section
  "Experiments").  The page gives no formula; an element-wise ratio is unbounded
  near zeros and could not give the page's values of a few unit roundoffs, so
  the error is normalised by the tensor's largest magnitude.
* ``rel_rms(x, ref) = ||x - ref||_2 / max(||ref||_2, 1e-30)`` -- the relative
  L2 / relative RMS error of the fla issue #1550 page ("Reproduction and
  evidence") and of the cuLA issue #126 page (its ``rel_l2``).
* ``rel_rms_per_head`` -- the same relative RMS taken separately for every
  (sequence, head) pair, the per-head breakdown the cuLA issue #126 page asks
  for ("Expected behavior / suggested coverage"); ``worst_head_rel_rms`` is its
  maximum.
"""
from __future__ import annotations

import numpy as np


def _pair(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise ValueError(f"shape mismatch {x.shape} vs {ref.shape}")
    return x, ref


def max_rel(x, ref) -> float:
    x, ref = _pair(x, ref)
    if x.size == 0:
        return 0.0
    den = np.max(np.abs(ref))
    num = np.max(np.abs(x - ref))
    if not np.isfinite(num):
        return float("inf")
    return float(num / max(den, 1e-300))


def rel_rms(x, ref) -> float:
    x, ref = _pair(x, ref)
    if x.size == 0:
        return 0.0
    num = np.linalg.norm((x - ref).ravel())
    if not np.isfinite(num):
        return float("inf")
    return float(num / max(np.linalg.norm(ref.ravel()), 1e-30))


def rel_rms_per_head(x, ref, cu_seqlens=None, token_major: bool = True) -> np.ndarray:
    """rel_rms of every (sequence, head) slice, as an (N, H) float64 array.

    token_major=True: tensors laid out (B, T, H, ...) -- per-token outputs and
    gradients; with ``cu_seqlens`` (packed, B == 1) sequence n is the token range
    [cu[n], cu[n+1]).  token_major=False: tensors laid out (N, H, ...) -- states.
    """
    x, ref = _pair(x, ref)
    if not token_major:
        if x.ndim < 2:
            raise ValueError("state tensors must be (N, H, ...)")
        N, H = x.shape[:2]
        return np.array([[rel_rms(x[n, h], ref[n, h]) for h in range(H)] for n in range(N)],
                        dtype=np.float64).reshape(N, H)
    if x.ndim < 3:
        raise ValueError("token-major tensors must be (B, T, H, ...)")
    B, T, H = x.shape[:3]
    if cu_seqlens is None:
        return np.array([[rel_rms(x[b, :, h], ref[b, :, h]) for h in range(H)] for b in range(B)],
                        dtype=np.float64).reshape(B, H)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if B != 1 or cu.ndim != 1 or cu.size < 1 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("packed tensors need B == 1 and monotone offsets from 0 to T")
    N = cu.size - 1
    return np.array([[rel_rms(x[0, cu[n]:cu[n + 1], h], ref[0, cu[n]:cu[n + 1], h]) for h in range(H)]
                     for n in range(N)], dtype=np.float64).reshape(N, H)


def worst_head_rel_rms(x, ref, cu_seqlens=None, token_major: bool = True) -> float:
    """The largest per-(sequence, head) rel_rms (0 for an empty tensor)."""
    per = rel_rms_per_head(x, ref, cu_seqlens, token_major)
    return float(per.max()) if per.size else 0.0
