"""Number formats the path reads and writes, defined from first principles.

  BF16   1 sign, 8 exponent (bias 127), 7 stored mantissa bits: the upper half
         of an IEEE binary32. Rounding is to nearest, ties to even mantissa,
         from the exact (here: float64) value in one step.
  E4M3   OCP FP8 "E4M3FN": 1 sign, 4 exponent (bias 7), 3 mantissa bits, no
         infinities, 0x7F / 0xFF are NaN, largest finite 448. The block scales
         of NVFP4 use it (vLLM API docs, prepare_trtllm_nvfp4, the quantizer
         `_quantize_nvfp4_global_scale`: scales stored as float8e4nv).
  E2M1   FP4 with the magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}, code = index in
         that list, bit 3 = sign; rounding to nearest with ties to the even
         code, saturating at 6 (same quantizer's comment on its code step).

Test infrastructure: only tests/, the smoke check and the benchmark's CPU
baseline import this package.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# BF16
# ----------------------------------------------------------------------------

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
_BF16_MIN_NORMAL_EXP = -126


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode BF16 bit patterns (uint16) exactly to float64."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u32.view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest BF16 value, ties to even, in one step.

    Returns the rounded values as float64. A BF16 value has 8 significant bits,
    so within the binade [2^e, 2^(e+1)) the spacing is 2^(e-7); below the
    smallest normal 2^-126 the spacing stays 2^-133 (subnormals). Magnitudes
    that round past the largest finite value become infinities; NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x) & (x != 0)
    xf = x[fin]
    # exponent of the leading bit: |x| in [2^e, 2^(e+1))
    _, e2 = np.frexp(xf)          # xf = m * 2^e2 with 0.5 <= |m| < 1
    e = np.maximum(e2 - 1, _BF16_MIN_NORMAL_EXP)
    quantum = np.ldexp(1.0, e - 7)
    q = np.rint(xf / quantum)     # division by a power of two is exact; rint is ties-to-even
    r = q * quantum
    r[np.abs(r) > BF16_MAX] = np.inf * np.sign(r[np.abs(r) > BF16_MAX])
    out[fin] = r
    return out


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to BF16 (one rounding) and return the bit patterns.

    NaN becomes the quiet NaN 0x7FC0 (sign kept)."""
    r = round_bf16(x)
    nan = np.isnan(r)
    r32 = r.astype(np.float32)    # exact: r is a BF16 value or +-inf
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        sign = (np.signbit(r[nan])).astype(np.uint16) << np.uint16(15)
        bits[nan] = np.uint16(0x7FC0) | sign
    return bits


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of BF16 values at the magnitude of x (float64 in, float64 out):
    2^(e-7) for |x| in [2^e, 2^(e+1)), and 2^-133 below the normal range."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e2 = np.frexp(np.where(x > 0, x, 1.0))
    e = np.where(x > 0, np.maximum(e2 - 1, _BF16_MIN_NORMAL_EXP), _BF16_MIN_NORMAL_EXP)
    return np.ldexp(1.0, e - 7)


# ----------------------------------------------------------------------------
# E4M3 (FN)
# ----------------------------------------------------------------------------


def e4m3_value(code: int) -> float:
    """Value of a non-negative E4M3 code 0x00..0x7E (0x7F is NaN)."""
    if not 0 <= code <= 0x7E:
        raise ValueError("not a finite non-negative E4M3 code")
    exp = code >> 3
    man = code & 7
    if exp == 0:
        return man * 2.0 ** -9            # subnormal: man/8 * 2^(1-7)
    return (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3_VALUES = np.array([e4m3_value(c) for c in range(0x7F)], dtype=np.float64)
E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Decode E4M3 bytes to float64 (sign bit 0x80; 0x7F/0xFF decode to NaN)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = c & np.uint8(0x7F)
    v = np.where(mag == 0x7F, np.nan, E4M3_VALUES[np.minimum(mag, 0x7E)])
    return np.where(c & np.uint8(0x80), -v, v)


def e4m3_encode_satfinite(x: np.ndarray) -> np.ndarray:
    """Round float values to E4M3 codes: nearest value, ties to the even code,
    magnitudes above 448 saturate to 448 (0x7E / 0xFE), the sign bit follows
    the sign of the input (-0.0 gives 0x80), NaN gives 0x7F.

    The decision compares |x| with the midpoint of its two neighbouring
    representable values; midpoints of E4M3 neighbours are exact in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    lo = np.searchsorted(E4M3_VALUES, a, side="right") - 1   # largest value <= a
    lo = np.clip(lo, 0, 0x7E)
    hi = np.minimum(lo + 1, 0x7E)
    mid = (E4M3_VALUES[lo] + E4M3_VALUES[hi]) * 0.5
    pick_hi = (a > mid) | ((a == mid) & (lo % 2 == 1))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = code.astype(np.uint8) | (np.signbit(x).astype(np.uint8) << np.uint8(7))
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


# ----------------------------------------------------------------------------
# E2M1
# ----------------------------------------------------------------------------

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_encode(q: np.ndarray) -> np.ndarray:
    """FP4 code of each value: the magnitude goes to the nearest grid value
    (ties to the even code, saturating at 6), and bit 3 is set exactly when the
    value is negative (so a small negative value that rounds to zero keeps its
    sign bit, and -0.0 does not). NaN gives code 0.
    """
    q = np.asarray(q, dtype=np.float64)
    a = np.abs(q)
    lo = np.searchsorted(E2M1_VALUES, a, side="right") - 1
    lo = np.clip(lo, 0, 7)
    hi = np.minimum(lo + 1, 7)
    mid = (E2M1_VALUES[lo] + E2M1_VALUES[hi]) * 0.5
    pick_hi = (a > mid) | ((a == mid) & (lo % 2 == 1))
    code = np.where(pick_hi, hi, lo)
    code = np.where(np.isnan(q), 0, code).astype(np.uint8)
    neg = (q < 0)
    return (code | (neg.astype(np.uint8) << np.uint8(3))).astype(np.uint8)


def e2m1_decode(code: np.ndarray) -> np.ndarray:
    c = np.asarray(code, dtype=np.uint8)
    v = E2M1_VALUES[c & np.uint8(7)]
    return np.where(c & np.uint8(8), -v, v)
