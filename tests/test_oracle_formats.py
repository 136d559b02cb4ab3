"""Pins of the oracle's number formats (BF16, E4M3, E2M1) against library
conversions, closed forms and the thresholds the quantizer page prints."""
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- BF16 ----

def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_torch_on_float32_inputs():
    g = np.random.default_rng(1)
    x = g.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    # exact ties: low 16 bits 0x8000, with even and odd kept mantissas
    u = g.integers(0x3F000000, 0x40800000, size=20_000, dtype=np.uint32)
    ties = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    near = np.concatenate([np.nextafter(ties, np.float32(np.inf)), np.nextafter(ties, np.float32(-np.inf))])
    sub = (g.integers(1, 1 << 23, size=5000, dtype=np.uint32)).view(np.float32)  # FP32 subnormals
    big = np.array([3.3e38, -3.3e38, 3.39e38, 1e-45, -1e-45, 0.0, -0.0], dtype=np.float32)
    allx = np.concatenate([x, ties, -ties, near, sub, big]).astype(np.float32)
    got = O.f64_to_bf16_bits(allx.astype(np.float64))
    np.testing.assert_array_equal(got, _torch_bf16_bits(allx))


def test_bf16_rounds_once_from_float64():
    # A value just above a BF16 midpoint that FP32 cannot hold: rounding via
    # FP32 first would land on the midpoint and then go to even (down).
    lo = 1.0                       # BF16 neighbours 1.0 and 1.0078125
    mid = lo + 2.0 ** -8
    above = mid + 2.0 ** -40
    below = mid - 2.0 ** -40
    assert np.float32(above) == np.float32(mid)        # FP32 would lose it
    assert O.round_bf16(np.array([above]))[0] == 1.0078125
    assert O.round_bf16(np.array([below]))[0] == 1.0
    assert O.round_bf16(np.array([mid]))[0] == 1.0     # tie -> even mantissa
    odd = 1.0078125
    assert O.round_bf16(np.array([odd + 2.0 ** -8]))[0] == 1.015625  # tie -> even (up)


def test_bf16_overflow_and_specials():
    maxv = (2 - 2.0 ** -7) * 2.0 ** 127
    half_ulp = 2.0 ** 119
    r = O.round_bf16(np.array([maxv, maxv + half_ulp * 0.999, maxv + half_ulp, -maxv - half_ulp, np.inf, np.nan, 0.0, -0.0]))
    assert r[0] == maxv and r[1] == maxv
    assert r[2] == np.inf and r[3] == -np.inf and r[4] == np.inf
    assert np.isnan(r[5]) and r[6] == 0.0 and np.signbit(r[7])
    bits = O.f64_to_bf16_bits(np.array([np.nan, -np.nan, -0.0]))
    assert bits[0] == 0x7FC0 and bits[1] == 0xFFC0 and bits[2] == 0x8000


def test_bf16_decode_matches_torch():
    g = np.random.default_rng(2)
    bits = g.integers(0, 1 << 16, size=50_000, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_bits_to_f64(bits)
    same = (got == t) | (np.isnan(got) & np.isnan(t))
    assert same.all()


def test_bf16_ulp_closed_forms():
    np.testing.assert_array_equal(O.bf16_ulp(np.array([1.0, 1.99, 2.0, 0.75, 2.0 ** -126, 2.0 ** -130])),
                                  [2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -8, 2.0 ** -133, 2.0 ** -133])


# ---------------------------------------------------------------- E4M3 ----

def test_e4m3_table_closed_forms():
    v = O.E4M3_VALUES
    assert v.size == 127 and np.all(np.diff(v) > 0)
    assert v[0x00] == 0.0 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x08] == 2.0 ** -6 and v[0x30] == 0.5 and v[0x38] == 1.0
    assert v[0x40] == 2.0 and v[0x7E] == 448.0 and v[0x78] == 256.0 and v[0x77] == 240.0


def test_e4m3_roundtrip_every_code():
    codes = np.arange(0x7F, dtype=np.uint8)
    np.testing.assert_array_equal(O.e4m3_encode_satfinite(O.e4m3_decode(codes)), codes)
    neg = codes | np.uint8(0x80)
    np.testing.assert_array_equal(O.e4m3_encode_satfinite(O.e4m3_decode(neg)), neg)
    assert O.e4m3_encode_satfinite(np.array([np.nan]))[0] == 0x7F
    assert np.isnan(O.e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def test_e4m3_matches_torch_below_saturation():
    g = np.random.default_rng(3)
    x = np.concatenate([
        g.uniform(0, 464, 100_000), g.uniform(0, 0.05, 50_000),
        (O.E4M3_VALUES[:-1] + O.E4M3_VALUES[1:]) / 2,           # every midpoint
        np.nextafter((O.E4M3_VALUES[:-1] + O.E4M3_VALUES[1:]) / 2, 0),
        np.nextafter((O.E4M3_VALUES[:-1] + O.E4M3_VALUES[1:]) / 2, 1e9),
    ]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode_satfinite(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_e4m3_saturates():
    x = np.array([448.0, 449.0, 464.0, 479.9, 480.0, 1e6, np.inf])
    np.testing.assert_array_equal(O.e4m3_encode_satfinite(x), [0x7E] * 7)
    np.testing.assert_array_equal(O.e4m3_encode_satfinite(-x), [0xFE] * 7)
    # underflow: half the smallest subnormal ties to zero, just above goes up
    assert O.e4m3_encode_satfinite(np.array([2.0 ** -10]))[0] == 0
    assert O.e4m3_encode_satfinite(np.array([2.0 ** -10 * 1.0001]))[0] == 1
    assert O.e4m3_encode_satfinite(np.array([3 * 2.0 ** -10]))[0] == 2   # 1.5 -> even code 2


# ---------------------------------------------------------------- E2M1 ----

def _load_thresholds():
    rows = []
    with open(os.path.join(GOLDEN, "e2m1_thresholds.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            v, c = line.split()
            val = float.fromhex(v) if v.startswith("0x") else float(v)
            rows.append((val, int(c)))
    return rows


def test_e2m1_printed_thresholds():
    rows = _load_thresholds()
    vals = np.array([r[0] for r in rows], dtype=np.float32).astype(np.float64)
    want = np.array([r[1] for r in rows], dtype=np.uint8)
    np.testing.assert_array_equal(O.e2m1_encode(vals), want)
    np.testing.assert_array_equal(O.e2m1_encode(-vals[1:]), want[1:] | 8)


def test_e2m1_grid_and_sign():
    grid = O.E2M1_VALUES
    np.testing.assert_array_equal(O.e2m1_encode(grid), np.arange(8))
    np.testing.assert_array_equal(O.e2m1_decode(np.arange(16, dtype=np.uint8)),
                                  np.concatenate([grid, -grid]))
    assert O.e2m1_encode(np.array([-0.0]))[0] == 0           # -0.0 is not < 0
    assert O.e2m1_encode(np.array([-0.1]))[0] == 8           # negative, rounds to 0
    assert O.e2m1_encode(np.array([np.nan]))[0] == 0
    # brute force: nearest grid value, ties to the even code
    g = np.random.default_rng(4)
    q = g.uniform(-8, 8, 20_000)
    codes = O.e2m1_encode(q)
    for v, c in zip(q[:2000], codes[:2000]):
        d = [abs(abs(v) - gv) for gv in grid]
        best = min(d)
        cands = [i for i in range(8) if d[i] == best]
        exp = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
        assert (c & 7) == exp and bool(c & 8) == (v < 0)
