"""Pins of the oracle's output epilogue y = o / sqrt(mean(o^2) + eps) * w * silu(z)
(CPU only; "Research Sprint Day 2", "Building some intuition", step 7: normalise
per head, then gate): closed forms for constant rows and for silu at 0 and ln 3,
scale invariance, the unit RMS of the normalised row, and the weight acting per
column.
"""
import math

import numpy as np

import oracle


def test_constant_row_closed_form():
    o = np.full((1, 1, 1, 16), -3.0)
    z = np.full((1, 1, 1, 16), math.log(3.0))          # sigmoid(ln 3) = 3/4
    y = oracle.epilogue(o, z, eps=0.0)
    assert np.allclose(y, -1.0 * 0.75 * math.log(3.0), rtol=1e-15)
    assert np.all(oracle.epilogue(o, np.zeros_like(z), eps=0.0) == 0.0)   # silu(0) = 0


def test_scale_invariance_and_unit_rms():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((2, 5, 3, 64))
    z = rng.standard_normal((2, 5, 3, 64))
    y1 = oracle.epilogue(o, z, eps=0.0)
    y2 = oracle.epilogue(7.25 * o, z, eps=0.0)
    assert np.allclose(y1, y2, rtol=1e-14, atol=0)
    silu = z / (1.0 + np.exp(-z))
    n = y1 / silu
    assert np.allclose(np.sqrt(np.mean(n * n, axis=-1)), 1.0, rtol=1e-13)
    # eps shrinks the row: rms(n) = sqrt(m / (m + eps)), m = mean(o^2)
    m = np.mean(o * o, axis=-1)
    ne = oracle.epilogue(o, z, eps=0.5) / silu
    assert np.allclose(np.sqrt(np.mean(ne * ne, axis=-1)), np.sqrt(m / (m + 0.5)), rtol=1e-13)


def test_weight_scales_columns():
    rng = np.random.default_rng(4)
    o = rng.standard_normal((1, 3, 2, 32))
    z = rng.standard_normal((1, 3, 2, 32))
    w = rng.uniform(0.5, 2.0, size=32)
    assert np.allclose(oracle.epilogue(o, z, w), oracle.epilogue(o, z) * w, rtol=1e-15)
