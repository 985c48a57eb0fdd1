"""Pins of the error metrics every parity verdict goes through (oracle.compare).

The expected values are worked by hand from the definitions:
max_rel = max|x - ref| / max|ref| (the Day-1 page's "max relative error across
all elements", section "Experiments") and rel_rms = ||x - ref||_2 / ||ref||_2
(the fla issue #1550 page's relative RMS, "Reproduction and evidence"; the cuLA
issue #126 page's rel_l2).  Each case is chosen so that a plausible wrong
normaliser gives a different number; the last test applies the same pins to
such mutants and checks that every one of them is caught.
"""
import math

import numpy as np
import pytest

from oracle.compare import max_rel, rel_rms, rel_rms_per_head, worst_head_rel_rms


def test_max_rel_hand_values():
    assert max_rel([1, -2, 3], [1, -2, 5]) == pytest.approx(0.4, abs=0, rel=1e-15)
    assert max_rel([0, -4], [0, -5]) == pytest.approx(0.2, rel=1e-15)
    assert max_rel([1, 10], [2, 10]) == pytest.approx(0.1, rel=1e-15)
    # diff = (2, 0, 0, 8), max|ref| = 8 -> 1.0; the error is not averaged
    assert max_rel([[3, 0], [0, 0]], [[1, 0], [0, -8]]) == pytest.approx(1.0, rel=1e-15)
    assert max_rel([5.0], [5.0]) == 0.0


def test_rel_rms_hand_values():
    # ||(3, -4)|| / ||(0, 4)|| = 5 / 4
    assert rel_rms([3, 0], [0, 4]) == pytest.approx(1.25, rel=1e-15)
    # ||x|| != ||ref||: ||(0, 1)|| / ||(2, 0)|| = 0.5 (by ||x||: 1/sqrt(5); by ||ref||^2: 0.25)
    assert rel_rms([2, 1], [2, 0]) == pytest.approx(0.5, rel=1e-15)
    # a root of a sum, not a mean of ratios: ||(1, 1)|| / ||(1, 3)|| = sqrt(2 / 10)
    assert rel_rms([2, 4], [1, 3]) == pytest.approx(math.sqrt(0.2), rel=1e-15)
    # independent of the shape the elements are arranged in
    assert rel_rms(np.array([[2, 4]]), np.array([[1], [3]]).T) == pytest.approx(math.sqrt(0.2), rel=1e-15)
    assert rel_rms([1.0, 2.0], [1.0, 2.0]) == 0.0


def test_metrics_edge_cases():
    with pytest.raises(ValueError):
        max_rel([1, 2], [1, 2, 3])
    with pytest.raises(ValueError):
        rel_rms(np.zeros((2, 3)), np.zeros((3, 2)))
    assert max_rel([np.nan, 1.0], [1.0, 1.0]) == math.inf
    assert max_rel([np.inf, 1.0], [1.0, 1.0]) == math.inf
    assert rel_rms([np.nan, 1.0], [1.0, 1.0]) == math.inf
    assert rel_rms([1.0, -np.inf], [1.0, 1.0]) == math.inf
    assert max_rel([], []) == 0.0 and rel_rms([], []) == 0.0
    # a zero reference: the floor of the normaliser keeps the value finite and large
    assert rel_rms([1e-3], [0.0]) == pytest.approx(1e-3 / 1e-30)


def test_per_head_hand_values():
    # (B=2, T=2, H=2, D=1): head (b, h) holds x[b, :, h, 0]
    ref = np.zeros((2, 2, 2, 1))
    x = np.zeros((2, 2, 2, 1))
    ref[0, :, 0, 0] = (3, 4)        # error (0, 0)          -> 0
    ref[0, :, 1, 0] = (0, 2)
    x[0, :, 1, 0] = (1, 2)          # error (1, 0) / 2      -> 0.5
    ref[1, :, 0, 0] = (1, 0)
    x[1, :, 0, 0] = (1, 3)          # error (0, 3) / 1      -> 3
    ref[1, :, 1, 0] = (6, 8)
    x[1, :, 1, 0] = (6, 7)          # error (0, 1) / 10     -> 0.1
    x[0, :, 0, 0] = (3, 4)
    per = rel_rms_per_head(x, ref)
    np.testing.assert_allclose(per, [[0.0, 0.5], [3.0, 0.1]], rtol=1e-15)
    assert worst_head_rel_rms(x, ref) == pytest.approx(3.0, rel=1e-15)
    # the whole-tensor value hides the bad head: ||(1, 3, 1)|| / ||(3, 4, 2, 1, 6, 8)||
    assert rel_rms(x, ref) == pytest.approx(math.sqrt(11.0 / 130.0), rel=1e-15)


def test_per_head_packed_and_states():
    # packed: one row of T = 5, sequences [0, 2) and [2, 5), H = 1
    ref = np.array([1.0, 0.0, 0.0, 0.0, 2.0]).reshape(1, 5, 1, 1)
    x = np.array([1.0, 1.0, 0.0, 0.0, 2.0]).reshape(1, 5, 1, 1)
    per = rel_rms_per_head(x, ref, cu_seqlens=[0, 2, 5])
    np.testing.assert_allclose(per, [[1.0], [0.0]], rtol=1e-15)
    with pytest.raises(ValueError):
        rel_rms_per_head(x, ref, cu_seqlens=[0, 2, 4])
    # states (N, H, Dk, Dv)
    S_ref = np.ones((2, 1, 2, 2))
    S = S_ref.copy()
    S[1, 0, 0, 0] = 3.0             # error 2 / ||ones(2x2)|| = 1
    per = rel_rms_per_head(S, S_ref, token_major=False)
    np.testing.assert_allclose(per, [[0.0], [1.0]], rtol=1e-15)


def _mutants():
    """Wrong normalisers a metric could plausibly be written with."""
    def by_sq_norm(x, r):
        x, r = np.asarray(x, float), np.asarray(r, float)
        return float(np.linalg.norm((x - r).ravel()) / max(np.sum(r * r), 1e-30))

    def by_x_norm(x, r):
        x, r = np.asarray(x, float), np.asarray(r, float)
        return float(np.linalg.norm((x - r).ravel()) / max(np.linalg.norm(x.ravel()), 1e-30))

    def mean_of_ratios(x, r):
        x, r = np.asarray(x, float), np.asarray(r, float)
        return float(np.sqrt(np.mean((x - r) ** 2)) / max(np.sqrt(np.mean(r ** 2)), 1e-30) / np.sqrt(x.size))

    def max_signed(x, r):
        x, r = np.asarray(x, float), np.asarray(r, float)
        return float(np.max(np.abs(x - r)) / max(np.max(r), 1e-300))

    def max_of_x(x, r):
        x, r = np.asarray(x, float), np.asarray(r, float)
        return float(np.max(np.abs(x - r)) / max(np.max(np.abs(x)), 1e-300))

    def elementwise(x, r):
        x, r = np.asarray(x, float), np.asarray(r, float)
        return float(np.max(np.abs(x - r) / np.maximum(np.abs(r), 1e-300)))

    return {"rel_rms": [by_sq_norm, by_x_norm, mean_of_ratios],
            "max_rel": [max_signed, max_of_x, elementwise]}


def _pins_hold(fn, which) -> bool:
    try:
        if which == "max_rel":
            cases = [([1, -2, 3], [1, -2, 5], 0.4), ([0, -4], [0, -5], 0.2), ([1, 10], [2, 10], 0.1)]
        else:
            cases = [([3, 0], [0, 4], 1.25), ([2, 1], [2, 0], 0.5), ([2, 4], [1, 3], math.sqrt(0.2))]
        return all(abs(fn(x, r) - e) <= 1e-12 * e for x, r, e in cases)
    except (ZeroDivisionError, FloatingPointError, ValueError):
        return False


def test_pins_catch_planted_wrong_normalisers():
    assert _pins_hold(max_rel, "max_rel") and _pins_hold(rel_rms, "rel_rms")
    for which, fns in _mutants().items():
        for fn in fns:
            with np.errstate(all="ignore"):
                assert not _pins_hold(fn, which), f"{which} mutant {fn.__name__} passed the pins"
