"""Error metrics used to compare a result with the oracle -- TEST INFRASTRUCTURE.

Both are computed in float64 over a whole tensor (or a slice the caller picks).

* ``max_rel(x, ref) = max|x - ref| / max|ref|`` -- the "max relative error
  across all elements" of the Day-1 page ("Research Sprint Day 1", section
  "Experiments").  The page gives no formula; an element-wise ratio is unbounded
  near zeros and could not give the page's values of a few unit roundoffs, so
  the error is normalised by the tensor's largest magnitude.
* ``rel_rms(x, ref) = ||x - ref||_2 / max(||ref||_2, 1e-30)`` -- the relative
  L2 / relative RMS error of the fla issue #1550 page ("Reproduction and
  evidence") and of the cuLA issue #126 page (its ``rel_l2``).
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
