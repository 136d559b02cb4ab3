"""Checks of the router projection shared by the GPU parity tests and the CPU
test that shows they catch a projection which drops a weight plane.

The projection is defined with FP32 weights and FP32 accumulation
(TensorRT-LLM PR #21356, "Add the Muse Spark Open decoder fast paths",
description, Triton kernel "Router projection"); the same page's "Not in this
PR" names the BF16x3 split of the weights that the HIP path uses. Two kinds of
input pin it:

* one-hot rows (one entry +-2^m, the rest zero): the exact dot product is
  2^m * W[e, i], so every logit must equal RN32(scale * 2^m * W[e, i]) bit
  for bit, whatever the accumulation order;
* same-sign rows (h >= 0) against positive weights whose third BF16 plane is
  positive: nothing cancels, so a projection that loses part of the weight
  errs by the lost part's full sum, far beyond the accumulation bound.

No torch here: the CPU suite imports this module.
"""
from __future__ import annotations

import numpy as np

import oracle as O
import workloads as wl

# Logit bound (parity rule R2): |GPU - oracle| <= 2^-19 |scale| sum_i |h_i W[e,i]|
# plus one FP32 rounding of the result. 2^-19 is 32 units of 2^-24 at the
# scale of sum|hW|: an FP32 accumulation of exact products stays a few units
# away (measured up to ~12 units), while a weight that keeps only two of its
# three BF16 planes loses up to 2^-17 of each product.
R2_UNITS = 32.0


def logit_bound(magnitude, logits_ref):
    """Elementwise R2 bound; magnitude = |scale| sum|h W| from the oracle."""
    return R2_UNITS * 2.0 ** -24 * np.asarray(magnitude, np.float64) + \
        2.0 ** -24 * np.abs(np.asarray(logits_ref, np.float32).astype(np.float64))


def r2_units(lg_gpu, lg_ref, magnitude):
    """Errors in units of 2^-24 |scale| sum|hW| (float64 array)."""
    err = np.abs(np.asarray(lg_gpu, np.float32).astype(np.float64) - np.asarray(lg_ref, np.float32).astype(np.float64))
    return err / np.maximum(2.0 ** -24 * np.asarray(magnitude, np.float64), 1e-300)


def assert_r2(lg_gpu, lg_ref, magnitude, rows_ok=None, what="logits"):
    """Assert R2 on the rows selected by rows_ok (all rows if None); returns
    the largest error in units of 2^-24 sum|hW|."""
    lg_gpu = np.asarray(lg_gpu, np.float32)
    bound = logit_bound(magnitude, lg_ref)
    err = np.abs(lg_gpu.astype(np.float64) - np.asarray(lg_ref, np.float32).astype(np.float64))
    ok = np.ones(err.shape, bool) if rows_ok is None else np.asarray(rows_ok, bool)[:, None] & np.ones(err.shape, bool)
    bad = ok & ~(err <= bound)
    if bad.any():
        t, e = np.argwhere(bad)[0]
        raise AssertionError("%s: R2 fails at %d elements, e.g. [%d,%d] got %r want %r (%.1f units of 2^-24 sum|hW|)" % (
            what, int(bad.sum()), t, e, float(lg_gpu[t, e]), float(lg_ref[t, e]),
            float(r2_units(lg_gpu[t, e], lg_ref[t, e], magnitude[t, e]))))
    return float(r2_units(lg_gpu, lg_ref, magnitude)[ok].max()) if ok.any() else 0.0


# ---- one-hot rows ------------------------------------------------------------

def one_hot_rows(T: int, H: int, dtype: str, seed: int):
    """[T,H] rows with a single entry +-2^m (m in -4..4) at a seeded position;
    every column position occurs when T >= H. Returns (hidden, pos, val):
    hidden as BF16 bits (dtype 'bf16') or FP32 (dtype 'f32')."""
    g = np.random.default_rng(seed)
    pos = (np.arange(T) * 37 + g.integers(0, H)) % H
    val = (np.where(g.uniform(size=T) < 0.5, -1.0, 1.0) * 2.0 ** g.integers(-4, 5, size=T)).astype(np.float32)
    h = np.zeros((T, H), np.float32)
    h[np.arange(T), pos] = val
    return (wl.f32_to_bf16_bits(h) if dtype == "bf16" else h), pos, val


def one_hot_expected(W, pos, val, scale):
    """Closed form of the projection of one-hot rows: RN32(scale * v * W[e, i]).
    v is a power of two and scale * W has at most 48 significant bits, so the
    float64 product is exact and the only rounding is the final one."""
    W64 = np.asarray(W, np.float32).astype(np.float64)
    s = np.float64(np.float32(scale))
    return (s * val.astype(np.float64)[:, None] * W64[:, pos].T).astype(np.float32)


def full_mantissa_weight(E: int, H: int, seed: int, std: float = 0.01) -> np.ndarray:
    """FP32 weights N(0, std) whose significands use all 24 bits: the low 8
    bits (the third BF16 plane's share) are forced nonzero."""
    g = np.random.default_rng(seed)
    W = (g.standard_normal((E, H)) * std).astype(np.float32)
    u = W.view(np.uint32)
    u |= (g.integers(1, 256, size=u.shape).astype(np.uint32))   # low byte nonzero
    return W


# ---- same-sign rows ----------------------------------------------------------

def positive_third_plane_weight(E: int, H: int, seed: int) -> np.ndarray:
    """Positive FP32 weights with 24 significant bits whose BF16x3 split
    (round to nearest even at each plane) has three positive planes.

    W = 2^e (1.a + 2^-9 1.b + 2^-18 1.c) with a, b 7-bit and c 5-bit fields:
    bit 8 and bit 17 below the leading one are zero, so each plane rounds
    down and leaves a positive remainder; the third plane is 2^(e-18) 1.c,
    between 2^-19 and 2^-17 of W. Exponents e in -9..-5 (values ~0.002-0.06).
    """
    g = np.random.default_rng(seed)
    e = g.integers(-9, -4, size=(E, H))
    a = g.integers(0, 128, size=(E, H))
    b = g.integers(0, 128, size=(E, H))
    c = g.integers(0, 32, size=(E, H))
    sig = (1 << 23) | (a << 16) | (1 << 14) | (b << 7) | (1 << 5) | c   # 24-bit integer significand
    W = (sig.astype(np.float64) * 2.0 ** (e - 23)).astype(np.float32)
    assert np.array_equal(W.astype(np.float64), sig.astype(np.float64) * 2.0 ** (e - 23))
    return W


def nonnegative_rows(T: int, H: int, dtype: str, seed: int, sparse: int = 0):
    """Rows with h >= 0: |N(0,1)| (dense), or `sparse` entries 2^m (m in -3..3)
    at seeded positions and zeros elsewhere."""
    g = np.random.default_rng(seed)
    if sparse:
        h = np.zeros((T, H), np.float32)
        for t in range(T):
            p = g.choice(H, size=sparse, replace=False)
            h[t, p] = 2.0 ** g.integers(-3, 4, size=sparse)
    else:
        h = np.abs(g.standard_normal((T, H))).astype(np.float32)
    return wl.f32_to_bf16_bits(h) if dtype == "bf16" else h


# ---- BF16 planes (used by the CPU test to model a two-plane projection) -----

def bf16_planes(W: np.ndarray, n: int):
    """The first n BF16 planes of the round-to-nearest-even split of FP32 W
    (each plane the BF16 rounding of what the previous ones left), as FP32."""
    rest = np.asarray(W, np.float32).copy()
    planes = []
    for _ in range(n):
        p = O.bf16_bits_to_f64(wl.f32_to_bf16_bits(rest)).astype(np.float32)
        planes.append(p)
        rest = (rest - p).astype(np.float32)
    return planes
