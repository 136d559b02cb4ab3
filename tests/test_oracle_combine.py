"""Pins of the combine oracle: power-of-two rows (exact norm) with power-of-two
weights give exact sums; invalid slots are never read; constant rows pin the
variance over x; row-permutation invariance and weight linearity."""
import numpy as np
import pytest

import oracle as O
import workloads as wl


def _bits(v):
    return wl.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def test_power_of_two_rows_and_weights_are_exact():
    g = np.random.default_rng(30)
    T, k, H = 6, 4, 64
    R = T * k
    ex = g.integers(-4, 4, size=(R, 1))
    signs = g.choice([-1.0, 1.0], size=(R, H))
    rows = signs * 2.0 ** ex
    gain = O.round_bf16(g.uniform(0.5, 1.5, H)).astype(np.float32)       # BF16-exact gains
    w = (2.0 ** g.integers(-3, 1, size=(T, k))).astype(np.float32)
    slots = np.arange(R).reshape(T, k)
    out, mag = O.combine(_bits(rows), slots, w, gain, 0.0, 0.0)
    z = signs * gain[None, :].astype(np.float64)                          # normalised rows, exact
    exact = (w.reshape(R, 1).astype(np.float64) * z).reshape(T, k, H).sum(1)
    np.testing.assert_array_equal(out, O.f64_to_bf16_bits(exact))


def test_single_slot_unit_weight_is_the_rounded_norm():
    g = np.random.default_rng(31)
    R, H = 10, 128
    rows = _bits(g.standard_normal((R, H)) * 3)
    gain = g.uniform(0.5, 1.5, H).astype(np.float32)
    out, _ = O.combine(rows, np.arange(R).reshape(R, 1), np.ones((R, 1), np.float32), gain, 0.0, 1e-6)
    np.testing.assert_array_equal(out, O.f64_to_bf16_bits(O.rmsnorm_bf16(rows, gain, 0.0, 1e-6)))


def test_constant_rows_pin_the_variance_over_the_row():
    H = 16
    gain = np.linspace(0.5, 1.5, H).astype(np.float32)
    rows = _bits(np.array([[0.25] * H, [-7.0] * H]))
    out, _ = O.combine(rows, np.array([[0], [1]]), np.ones((2, 1), np.float32), gain, 0.0, 0.0)
    want = O.f64_to_bf16_bits(np.stack([gain, -gain]).astype(np.float64))
    np.testing.assert_array_equal(out, want)


def test_invalid_slots_are_never_read():
    w_ = wl.WORKLOADS["tiny"]
    eo = wl.expert_out(w_)
    slots, invalid_rows = wl.combine_slots(w_)
    assert len(invalid_rows) == 6
    tw = wl.routing_weights(w_)
    gain = wl.combine_gain(w_)
    eo_nan = eo.copy()
    eo_nan[invalid_rows] = wl.BF16_NAN
    out_nan, _ = O.combine(eo_nan, slots, tw, gain, 0.0, w_.eps)
    out_fin, _ = O.combine(eo, slots, tw, gain, 0.0, w_.eps)
    np.testing.assert_array_equal(out_nan, out_fin)
    assert not np.isnan(O.bf16_bits_to_f64(out_nan)).any()
    # out-of-range slots are invalid too, and a token with no valid slot is +0.0
    s2 = slots.copy()
    s2[0] = [-1, w_.R, w_.R + 5, -7]
    out2, _ = O.combine(eo_nan, s2, tw, gain, 0.0, w_.eps)
    assert (out2[0] == 0).all()
    np.testing.assert_array_equal(out2[1:], out_nan[1:])


def test_row_permutation_invariance_and_weight_linearity():
    g = np.random.default_rng(32)
    T, k, H = 9, 3, 96
    R = T * k
    eo = _bits(g.standard_normal((R, H)))
    slots = g.permutation(R).reshape(T, k)
    w = g.uniform(0.1, 0.5, (T, k)).astype(np.float32)
    gain = g.uniform(0.5, 1.5, H).astype(np.float32)
    out, _ = O.combine(eo, slots, w, gain, 0.0, 1e-6)
    p = g.permutation(R)
    inv = np.argsort(p)
    out_p, _ = O.combine(eo[p], inv[slots], w, gain, 0.0, 1e-6)
    np.testing.assert_array_equal(out, out_p)
    out2, _ = O.combine(eo, slots, w * np.float32(4.0), gain, 0.0, 1e-6)
    np.testing.assert_array_equal(O.bf16_bits_to_f64(out2), 4.0 * O.bf16_bits_to_f64(out))
