"""Pins of the routing oracle: projection closed forms and exact sums, the
sigmoid against a library routine, brute-force sorted top-k with lowest-id
ties, renormalised-weight closed forms, and the validity mask."""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O
import workloads as wl


def test_projection_one_hot_is_the_weight_column():
    E, H = 7, 32
    g = np.random.default_rng(10)
    W = g.standard_normal((E, H)).astype(np.float32)
    h = np.zeros((H, H), dtype=np.float32)
    h[np.arange(H), np.arange(H)] = 1.0
    for scale in (1.0, 0.5, 3.0):
        lg, mag = O.router_logits(h, W, scale)
        np.testing.assert_array_equal(lg, (np.float64(scale) * W.T.astype(np.float64)).astype(np.float32))
    lg, _ = O.router_logits(g.standard_normal((4, H)).astype(np.float32), np.zeros((E, H), np.float32))
    assert (lg == 0).all()


def test_projection_matches_exact_sum_brute_force():
    g = np.random.default_rng(11)
    T, H, E = 5, 48, 6
    hb = wl.f32_to_bf16_bits(g.standard_normal((T, H)).astype(np.float32))
    W = (g.standard_normal((E, H)) * 0.05).astype(np.float32)
    hv = torch.from_numpy(hb.view(np.int16)).view(torch.bfloat16).float().numpy()  # decode by a library
    scale = 0.75
    lg, mag = O.router_logits(hb, W, scale)
    for t in range(T):
        for e in range(E):
            prods = [float(hv[t, i]) * float(W[e, i]) for i in range(H)]   # exact in float64
            exact = math.fsum(prods)
            assert lg[t, e] == np.float32(scale * exact)
            assert mag[t, e] == pytest.approx(scale * math.fsum(abs(p) for p in prods), rel=1e-12)


def test_sigmoid_against_library_and_closed_forms():
    x = np.array([0.0, 100.0, -100.0, 20.0, -20.0], dtype=np.float32)
    s = O.sigmoid_f32(x)
    assert s[0] == 0.5 and s[1] == 1.0 and s[3] == 1.0
    assert s[2] == np.float32(math.exp(-100.0) / (1 + math.exp(-100.0)))
    g = np.random.default_rng(12)
    lg = (g.standard_normal(100_000) * 4).astype(np.float32)
    np.testing.assert_array_equal(O.sigmoid_f32(lg), scipy.special.expit(lg.astype(np.float64)).astype(np.float32))
    # symmetry sigma(-l) = 1 - sigma(l), up to the two FP32 roundings
    assert np.abs(O.sigmoid_f32(-lg).astype(np.float64) + O.sigmoid_f32(lg) - 1).max() <= 2 ** -24


def _brute_topk(keys_row, k):
    E = len(keys_row)
    def rank(e):
        v = float(keys_row[e])
        return (1 if math.isnan(v) else 0, 0.0 if math.isnan(v) else -v, e)
    return sorted(range(E), key=rank)[:k]


@pytest.mark.parametrize("E,k", [(4, 1), (8, 3), (16, 4), (16, 16), (33, 8), (64, 22)])
def test_topk_brute_force_with_many_ties(E, k):
    g = np.random.default_rng(100 + E + k)
    T = 300
    # logits on a coarse grid and a bias taking few values: many equal keys
    lg = (g.integers(-4, 5, size=(T, E)) / 4.0).astype(np.float32)
    bias = (g.integers(-1, 2, size=E) / 8.0).astype(np.float32)
    keys = O.selection_keys(lg, bias)
    ids = O.topk_sorted(keys, k)
    for t in range(T):
        assert list(ids[t]) == _brute_topk(keys[t], k)


def test_topk_ties_go_to_lowest_id_and_zero_signs_tie():
    keys = np.zeros((1, 10), dtype=np.float32)
    np.testing.assert_array_equal(O.topk_sorted(keys, 4)[0], [0, 1, 2, 3])
    keys = np.array([[0.0, -0.0, 0.0, -0.0, 1.0]], dtype=np.float32)
    np.testing.assert_array_equal(O.topk_sorted(keys, 5)[0], [4, 0, 1, 2, 3])
    keys = np.array([[np.nan, 0.5, -np.inf, 0.5, np.nan]], dtype=np.float32)
    np.testing.assert_array_equal(O.topk_sorted(keys, 5)[0], [1, 3, 2, 0, 4])


def test_all_zero_logits_give_equal_weights():
    for k, E in [(4, 16), (8, 256), (22, 512)]:
        lg = np.zeros((3, E), dtype=np.float32)
        ids, w = O.route_from_logits(lg, np.zeros(E, np.float32), np.ones(3, np.uint8), k)
        np.testing.assert_array_equal(ids, np.tile(np.arange(k), (3, 1)))
        assert (w == np.float32(1.0) / np.float32(k)).all()


def test_bias_selects_but_does_not_weight():
    E, k = 12, 4
    lg = np.zeros((2, E), dtype=np.float32)
    bias = np.linspace(-0.2, 0.3, E).astype(np.float32)
    ids, w = O.route_from_logits(lg, bias, np.ones(2, np.uint8), k)
    np.testing.assert_array_equal(ids[0], [11, 10, 9, 8])          # largest bias first
    assert (w == np.float32(0.25)).all()                           # unbiased sigmoid(0) everywhere
    # unequal sigmoids: weight ratio follows the sigmoid, not sigmoid + bias
    lg = np.array([[2.0, 0.0, 0.0, 0.0]], dtype=np.float32)
    ids, w = O.route_from_logits(lg, np.array([0, 5, 0, 0], np.float32), np.ones(1, np.uint8), 2)
    np.testing.assert_array_equal(ids[0], [1, 0])
    s2 = 1 / (1 + math.exp(-2.0))
    assert w[0, 0] == pytest.approx(0.5 / (0.5 + s2), rel=1e-6)
    assert w[0, 1] == pytest.approx(s2 / (0.5 + s2), rel=1e-6)


def test_weights_sum_to_one_and_follow_pick_order():
    w_ = wl.WORKLOADS["decode"]
    lg = wl.tie_logits(w_)
    b = wl.bias(w_)
    ids, w = O.route_from_logits(lg, b, np.ones(w_.T, np.uint8), w_.k)
    assert np.abs(w.astype(np.float64).sum(1) - 1).max() <= w_.k * 2 ** -24
    keys = O.selection_keys(lg, b)
    kk = np.take_along_axis(keys, ids.astype(np.int64), axis=1)
    assert (np.diff(kk, axis=1) <= 0).all()                       # keys non-increasing
    assert all(len(set(r)) == w_.k for r in ids)                   # distinct ids


def test_tie_run_has_exact_ties_with_zero_bias():
    # The decode workload's grid logits produce equal keys when the bias is 0.
    w_ = wl.WORKLOADS["decode"]
    lg = wl.tie_logits(w_)
    keys = O.selection_keys(lg, np.zeros(w_.E, np.float32))
    ids = O.topk_sorted(keys, w_.k + 1)
    kk = np.take_along_axis(keys, ids.astype(np.int64), axis=1)
    ties = (np.diff(kk, axis=1) == 0)
    assert ties.any()
    for t in np.nonzero(ties.any(1))[0][:10]:
        assert list(ids[t, : w_.k]) == _brute_topk(keys[t], w_.k)


def test_mask_invalid_tokens_emit_nothing_and_nan_rows_are_ignored():
    g = np.random.default_rng(13)
    T, E, k = 40, 32, 6
    lg = g.standard_normal((T, E)).astype(np.float32)
    mask = (g.uniform(size=T) > 0.3).astype(np.uint8)
    b = (g.uniform(-0.1, 0.1, E)).astype(np.float32)
    ids, w = O.route_from_logits(lg, b, mask, k)
    assert (ids[mask == 0] == -1).all() and (w[mask == 0] == 0).all()
    assert (ids[mask == 1] >= 0).all()
    lg2 = lg.copy()
    lg2[mask == 0] = np.nan
    ids2, w2 = O.route_from_logits(lg2, b, mask, k)
    np.testing.assert_array_equal(ids, ids2)
    np.testing.assert_array_equal(w, w2)


def test_near_tie_detection():
    lg = np.array([[1.0, 1.0 + 2 ** -20, -3.0, -4.0], [3.0, 2.0, 1.0, 0.0]], dtype=np.float32)
    bound = np.full(lg.shape, 1e-4)
    near = O.key_gap_near_ties(lg, bound, np.zeros(4, np.float32), np.ones(2, np.uint8), 1)
    np.testing.assert_array_equal(near, [True, False])
