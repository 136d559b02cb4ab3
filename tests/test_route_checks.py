"""The projection pins of the GPU tests (one-hot rows exact, same-sign rows
within the tight R2 bound) reject a router that keeps only two of the three
BF16 planes of its FP32 weights, and accept the three-plane split.

TensorRT-LLM PR #21356, "Add the Muse Spark Open decoder fast paths",
description: the router projection keeps FP32 weights and FP32 accumulation
("Router projection"); a BF16x3 router is the split that keeps them exact
("Not in this PR"). Everything here runs on the CPU: the "projections" under
test are numpy models, evaluated exactly in float64 and rounded once.
"""
import numpy as np
import pytest

import oracle as O
import route_checks as RC
from oracle.route import hidden_to_f64


def _model_logits(hidden, planes, scale=1.0):
    """scale * sum_i h_i * (sum of the given weight planes)[e, i] rounded to
    FP32: exact products, a correctly rounded sum (math.fsum), then the scale
    (exact for the one-hot rows, where the sum has one term)."""
    import math
    h = hidden_to_f64(hidden)
    Wp = sum(p.astype(np.float64) for p in planes)
    s = np.float64(np.float32(scale))
    T, E = h.shape[0], Wp.shape[0]
    out = np.empty((T, E), np.float32)
    for t in range(T):
        nz = np.nonzero(h[t])[0]
        for e in range(E):
            out[t, e] = np.float32(s * math.fsum(h[t, nz] * Wp[e, nz]))
    return out


def test_weight_constructions():
    W = RC.full_mantissa_weight(8, 64, seed=1)
    assert ((W.view(np.uint32) & 0xFF) != 0).all()
    P = RC.positive_third_plane_weight(16, 64, seed=2)
    p0, p1, p2 = RC.bf16_planes(P, 3)
    assert (P > 0).all() and (p0 > 0).all() and (p1 > 0).all() and (p2 > 0).all()
    np.testing.assert_array_equal(p0.astype(np.float64) + p1 + p2, P.astype(np.float64))
    ratio = p2.astype(np.float64) / P
    assert ratio.min() >= 2.0 ** -19 * 0.99 and ratio.max() <= 2.0 ** -17
    # three RNE planes are exact for the random weights too
    q0, q1, q2 = RC.bf16_planes(W, 3)
    np.testing.assert_array_equal(q0.astype(np.float64) + q1 + q2, W.astype(np.float64))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_one_hot_pin_rejects_two_planes(dtype):
    T, H, E = 40, 64, 12
    hidden, pos, val = RC.one_hot_rows(T, H, dtype, seed=3)
    W = RC.full_mantissa_weight(E, H, seed=4)
    for scale in (1.0, 0.8125, -1.7):
        want = RC.one_hot_expected(W, pos, val, scale)
        np.testing.assert_array_equal(want, O.router_logits(hidden, W, scale)[0])
        three = _model_logits(hidden, RC.bf16_planes(W, 3), scale)
        np.testing.assert_array_equal(three, want)
        two = _model_logits(hidden, RC.bf16_planes(W, 2), scale)
        with pytest.raises(AssertionError):
            np.testing.assert_array_equal(two, want)
        assert (two != want).mean() > 0.9


@pytest.mark.parametrize("sparse", [0, 4])
def test_same_sign_pin_rejects_two_planes(sparse):
    T, H, E = 24, 256, 10
    hidden = RC.nonnegative_rows(T, H, "bf16", seed=5, sparse=sparse)
    W = RC.positive_third_plane_weight(E, H, seed=6)
    ref, mag = O.router_logits(hidden, W)
    three = _model_logits(hidden, RC.bf16_planes(W, 3))
    assert RC.assert_r2(three, ref, mag) <= 1.0          # exact sum, one rounding
    two = _model_logits(hidden, RC.bf16_planes(W, 2))
    with pytest.raises(AssertionError):
        RC.assert_r2(two, ref, mag)
    # every element fails, by about twice the bound
    units = RC.r2_units(two, ref, mag)
    assert units.min() > RC.R2_UNITS and np.median(units) > 1.5 * RC.R2_UNITS


def test_old_bound_was_blind_to_two_planes():
    """The bound the GPU test used before (n = 6 H/16 + 66 units) accepts a
    two-plane projection of the same-sign rows; the tight one does not."""
    T, H, E = 16, 1024, 8
    hidden = RC.nonnegative_rows(T, H, "bf16", seed=7)
    W = RC.positive_third_plane_weight(E, H, seed=8)
    ref, mag = O.router_logits(hidden, W)
    two = _model_logits(hidden, RC.bf16_planes(W, 2))
    old_units = (H // 16) * 6 + 66
    assert (RC.r2_units(two, ref, mag) < old_units).all()
    with pytest.raises(AssertionError):
        RC.assert_r2(two, ref, mag)
