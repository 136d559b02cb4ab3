"""moe_route against the oracle.

R1  the oracle's routing of the GPU's own logits equals the GPU's ids
    (bit-exact, order and -1s included) and weights (bit-exact expected; the
    contract allows 1e-5 relative);
R2  GPU logits within the FP32-accumulation bound of the oracle's float64
    projection;
R3  the oracle's routing of its own logits equals the GPU's ids except on
    tokens whose key gaps are within the propagated logit bound (near ties).
Plus the logits-in tie run, the validity mask with NaN rows, and edge shapes.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as wl
from gpu_helpers import dev, host, note, require_gpu

pytestmark = pytest.mark.gpu

m = pytest.importorskip("moe_token_routing_amd")

# Logit error bound: the projection accumulates in FP32 (three MFMA products
# per 16-wide K step, split-K partials added in order, one scale rounding), so
# its error is below n * 2^-24 * |scale| * sum|h*W| with n the longest chain
# of FP32 additions. n <= H/16*6 + 64 + 2 for every shape here; the bound
# below uses that n (plus one rounding of the result).
def logit_bound(magnitude, logits_ref, H):
    n = (H // 16) * 6 + 66
    return n * 2.0 ** -24 * magnitude + 2.0 ** -24 * np.abs(logits_ref.astype(np.float64))


def _route_gpu(hidden, W, bias, mask, k, scale=1.0):
    require_gpu()
    lg, ids, w = m.route(dev(hidden), dev(W), dev(bias), dev(mask), k, scale)
    torch.cuda.synchronize()
    return host(lg), host(ids), host(w)


def _check_r1(lg_gpu, ids, w, bias, mask, k, what):
    ids_o, w_o = O.route_from_logits(lg_gpu, bias, mask, k)
    np.testing.assert_array_equal(ids, ids_o, err_msg=what + ": R1 ids")
    rel = np.abs(w.astype(np.float64) - w_o) / np.maximum(np.abs(w_o), 1e-30)
    assert (rel <= 1e-5).all(), what + ": R1 weights beyond 1e-5"
    return float((w == w_o).mean())


def _check_projection(hidden, W, bias, mask, k, scale, rows, what):
    lg, ids, w = _route_gpu(hidden, W, bias, mask, k, scale)
    valid = mask[rows] != 0
    # R1 on the sampled rows (and their mask handling)
    exact_w = _check_r1(lg[rows], ids[rows], w[rows], bias, mask[rows], k, what)
    print("%s: bit-exact weight fraction %.6f" % (what, exact_w))
    # R2
    lg_ref, mag = O.router_logits(hidden[rows], W, scale)
    bound = logit_bound(mag, lg_ref, hidden.shape[1])
    err = np.abs(lg[rows].astype(np.float64) - lg_ref)
    okv = valid[:, None] & np.ones_like(err, dtype=bool)
    assert (err[okv] <= bound[okv]).all(), "%s: R2 max err/bound %.3g" % (what, (err[okv] / bound[okv]).max())
    # R3
    ids_ref, w_ref = O.route_from_logits(lg_ref, bias, mask[rows], k)
    near = O.key_gap_near_ties(lg_ref, bound, bias, mask[rows], k)
    differ = (ids[rows] != ids_ref).any(axis=1)
    assert not (differ & ~near).any(), "%s: R3 id mismatch outside the near-tie set" % what
    far = ~near & valid
    rel = np.abs(w[rows][far].astype(np.float64) - w_ref[far]) / np.abs(w_ref[far])
    assert (rel <= 1e-4).all()
    units = (err[okv] / (2.0 ** -24 * mag[okv])).max() if okv.any() else 0.0
    print("%s: max logit error %.2f x 2^-24 sum|hW|; near-tie tokens %d, differing %d" % (
        what, units, int(near.sum()), int(differ.sum())))


@pytest.mark.parametrize("name,T", [("tiny", None), ("decode", None), ("prefill", 300),
                                    ("large_e", 130), ("wide_k", 1000)])
def test_route_workloads(name, T):
    w = wl.WORKLOADS[name]
    T = w.T if T is None else T
    note("route %s T=%d" % (name, T))
    hidden = wl.hidden(w, T)
    W = wl.router_weight(w)
    bias = wl.bias(w)
    mask = wl.token_mask(w, T)
    _check_projection(hidden, W, bias, mask, w.k, 1.0, np.arange(T), name)


@pytest.mark.parametrize("name", ["prefill", "large_e", "wide_k"])
def test_route_full_size_sampled(name):
    w = wl.WORKLOADS[name]
    note("route %s full" % name)
    hidden = wl.hidden(w)
    W = wl.router_weight(w)
    bias = wl.bias(w)
    mask = wl.token_mask(w)
    g = np.random.default_rng(9)
    rows = np.unique(np.concatenate([g.choice(w.T, 400, replace=False), [0, w.T - 1]]))
    _check_projection(hidden, W, bias, mask, w.k, 1.0, rows, name + "-full")


def test_route_scale_and_ragged_shapes():
    g = np.random.default_rng(60)
    # below 4096 tokens the projection splits the weights in registers, from
    # 4096 it reads planes split by a kernel of their own: both with a ragged
    # token tile and a padded expert tile
    # (token tiles of 32, 64 or 128 rows by count: 3000 takes 128-row tiles
    # with the in-register split)
    for T, H, E, k in [(1, 16, 1, 1), (3, 48, 5, 5), (70, 1040, 200, 6), (129, 256, 64, 32), (33, 4096, 4096, 8),
                       (9, 16384, 64, 4), (3000, 512, 256, 8), (4100, 272, 300, 8)]:
        note("route ragged T=%d H=%d E=%d k=%d" % (T, H, E, k))
        hidden = wl.f32_to_bf16_bits(g.standard_normal((T, H)).astype(np.float32))
        W = (g.standard_normal((E, H)) * 0.02).astype(np.float32)
        bias = g.uniform(-0.05, 0.05, E).astype(np.float32)
        mask = (g.uniform(size=T) > 0.1).astype(np.uint8)
        mask[0] = 1
        _check_projection(hidden, W, bias, mask, k, 0.75, np.arange(T), "ragged %d/%d/%d/%d" % (T, H, E, k))


@pytest.mark.parametrize("T", [300, 4100])
def test_route_fp32_input(T):
    """FP32 hidden states (three input planes): 300 tokens split the weights
    in registers, 4100 read the split kernel's planes."""
    w = wl.WORKLOADS["tiny"]
    g = np.random.default_rng(61)
    hidden = (g.standard_normal((T, w.H)) * 3).astype(np.float32)
    W = wl.router_weight(w)
    bias = wl.bias(w)
    mask = np.ones(T, np.uint8)
    _check_projection(hidden, W, bias, mask, w.k, 1.0, np.arange(T), "fp32 input %d" % T)


def test_route_logits_in_tie_run():
    """Decode workload: 25% of tokens carry logits on a 2^-8 grid. With zero
    bias they produce exact key ties, which must go to the lowest id."""
    w = wl.WORKLOADS["decode"]
    require_gpu()
    for seed_shift in range(4):
        lg = wl.tie_logits(w)
        if seed_shift:
            lg = np.roll(lg, seed_shift * 37, axis=1)
        for bias in (np.zeros(w.E, np.float32), wl.bias(w),
                     (np.random.default_rng(seed_shift).integers(-2, 3, w.E) / 64).astype(np.float32)):
            mask = np.ones(w.T, np.uint8)
            mask[5] = 0
            note("route logits-in ties shift=%d" % seed_shift)
            lg_d = dev(lg)
            _, ids, wt = m.route(None, None, dev(bias), dev(mask), w.k, logits=lg_d)
            ids, wt = host(ids), host(wt)
            ids_o, w_o = O.route_from_logits(lg, bias, mask, w.k)
            np.testing.assert_array_equal(ids, ids_o)
            np.testing.assert_array_equal(wt, w_o)
            np.testing.assert_array_equal(host(lg_d), lg)      # logits are an input here


def test_route_exact_ties_all_equal():
    require_gpu()
    for E, k in [(16, 4), (256, 8), (512, 22), (2560, 8), (4096, 32)]:
        lg = np.zeros((3, E), np.float32)
        lg[1, ::3] = 0.5
        lg[2] = -0.0
        bias = np.zeros(E, np.float32)
        bias[7 % E] = -0.0
        mask = np.ones(3, np.uint8)
        _, ids, wt = m.route(None, None, dev(bias), dev(mask), k, logits=dev(lg))
        ids_o, w_o = O.route_from_logits(lg, bias, mask, k)
        np.testing.assert_array_equal(host(ids), ids_o)
        np.testing.assert_array_equal(host(wt), w_o)


@pytest.mark.parametrize("E,k", [(512, 22), (512, 11), (300, 12), (128, 16), (64, 32), (40, 13)])
def test_route_logits_in_ties_many_picks(E, k):
    """From 12 picks the selection searches the k-th largest key bit by bit
    (below, it takes k rounds): logits on a coarse grid (many exact key
    ties, across the k-th place too), a few NaN logits (keys below every
    number) and a coarse bias, against the oracle bit for bit."""
    require_gpu()
    g = np.random.default_rng(E + k)
    T = 64
    lg = (g.integers(-6, 7, size=(T, E)) / 4).astype(np.float32)
    lg[g.uniform(size=(T, E)) < 0.02] = np.nan
    lg[3] = 0.0                                               # one token all equal
    bias = (g.integers(-2, 3, E) / 32).astype(np.float32)
    mask = np.ones(T, np.uint8)
    mask[7] = 0
    note("route logits-in ties E=%d k=%d" % (E, k))
    _, ids, wt = m.route(None, None, dev(bias), dev(mask), k, logits=dev(lg))
    ids_o, w_o = O.route_from_logits(lg, bias, mask, k)
    np.testing.assert_array_equal(host(ids), ids_o)
    np.testing.assert_array_equal(host(wt), w_o)


def test_route_mask_with_nan_rows():
    w = wl.WORKLOADS["prefill"]
    T = 256
    hidden = wl.hidden(w, T)
    mask = wl.token_mask(w, T)
    mask[::7] = 0
    W = wl.router_weight(w)
    bias = wl.bias(w)
    lg1, ids1, w1 = _route_gpu(hidden, W, bias, mask, w.k)
    hnan = hidden.copy()
    hnan[mask == 0] = wl.BF16_NAN
    lg2, ids2, w2 = _route_gpu(hnan, W, bias, mask, w.k)
    assert (ids2[mask == 0] == -1).all() and (w2[mask == 0] == 0).all()
    np.testing.assert_array_equal(ids1, ids2)
    np.testing.assert_array_equal(w1, w2)
    np.testing.assert_array_equal(lg1[mask == 1], lg2[mask == 1])


def test_route_is_deterministic():
    require_gpu()
    w = wl.WORKLOADS["decode"]
    hidden = dev(wl.hidden(w))
    W, bias, mask = dev(wl.router_weight(w)), dev(wl.bias(w)), dev(wl.token_mask(w))
    first = [host(t) for t in m.route(hidden, W, bias, mask, w.k)]
    for _ in range(5):
        again = [host(t) for t in m.route(hidden, W, bias, mask, w.k)]
        for a, b in zip(first, again):
            np.testing.assert_array_equal(a, b)
