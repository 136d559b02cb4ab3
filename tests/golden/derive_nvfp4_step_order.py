"""Derive tests/golden/nvfp4_step_order.txt: NVFP4 blocks whose scale byte or
codes depend on the order of the block quantiser's FP32 steps.

Source: vLLM API docs, vllm.models.muse_spark.nvidia.ops.prepare_trtllm_nvfp4,
`_quantize_nvfp4_global_scale` (the per-16-element block steps, in this
order): the block maximum times the FP32 constant 1/6, times the global
scale, converted to E4M3; the scale's value times the reciprocal of the
global scale; the reciprocal of that; each element times it, encoded as E2M1
by the printed thresholds. Readings: the page's approximate reciprocals are
IEEE correctly rounded FP32 reciprocals, and the FP32 -> E4M3 conversion
rounds to nearest even and saturates at 448.

Every step is carried out here in exact rational arithmetic (Python's
fractions), each FP32 rounding written out from the binary32 format's
definition, so the file can be checked by hand line by line. It uses neither
numpy nor the oracle. The block values were chosen so that a reordered or
fused chain changes the result: (gs * amax) * (1/6) or gs * amax / 6 in place
of gs * (amax * (1/6)), and gs / sf, gs * (1/sf) or 1 / (sf / gs) in place of
1 / (sf * (1/gs)). The file lists what each of those would give.

    python tests/golden/derive_nvfp4_step_order.py
"""
from __future__ import annotations

import os
from fractions import Fraction as Fr

HERE = os.path.dirname(os.path.abspath(__file__))


# ---- binary32 -----------------------------------------------------------------

def rn32(x: Fr) -> Fr:
    """Round a rational to the nearest binary32 value, ties to even
    (normal and subnormal range; the values here never overflow)."""
    if x == 0:
        return Fr(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fr(2) ** e > a:
        e -= 1
    e = max(e, -126)                       # subnormals share 2^-126's spacing
    ulp = Fr(2) ** (e - 23)
    q, r = divmod(a, ulp)
    q = int(q)
    if r > ulp / 2 or (r == ulp / 2 and q % 2 == 1):
        q += 1
    return sign * q * ulp


def f32_bits(x: Fr) -> int:
    """binary32 bit pattern of a value that is exactly representable."""
    if x == 0:
        return 0
    s = 0x80000000 if x < 0 else 0
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fr(2) ** e > a:
        e -= 1
    if e < -126:
        m = a / Fr(2) ** -149
        assert m.denominator == 1
        return s | int(m)
    m = a / Fr(2) ** (e - 23)
    assert m.denominator == 1 and (1 << 23) <= m < (1 << 24)
    return s | ((e + 127) << 23) | (int(m) - (1 << 23))


def from_f32_bits(b: int) -> Fr:
    s = -1 if b >> 31 else 1
    e = (b >> 23) & 0xFF
    m = b & 0x7FFFFF
    if e == 0:
        return s * m * Fr(2) ** -149
    return s * ((1 << 23) + m) * Fr(2) ** (e - 150)


def bf16(b: int) -> Fr:
    return from_f32_bits(b << 16)


# ---- E4M3 (OCP, "FN": no infinities, max 448) and E2M1 ------------------------

def e4m3_value(code: int) -> Fr:
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0:
        return Fr(m, 8) * Fr(2) ** -6
    return (1 + Fr(m, 8)) * Fr(2) ** (e - 7)


E4M3 = [(c, e4m3_value(c)) for c in range(0x7F)]       # 0x00 .. 0x7E (448)


def e4m3_rne_sat(x: Fr):
    """Nearest non-negative E4M3 value, ties to the even code, saturating at
    448. Returns (code, lower neighbour, upper neighbour)."""
    assert x >= 0
    if x >= 448:
        return 0x7E, E4M3[-1], E4M3[-1]
    lo = max((c for c in E4M3 if c[1] <= x), key=lambda c: c[1])
    hi = min((c for c in E4M3 if c[1] >= x), key=lambda c: c[1])
    if lo[1] == hi[1]:
        return lo[0], lo, hi
    mid = (lo[1] + hi[1]) / 2
    if x < mid or (x == mid and lo[0] % 2 == 0):
        return lo[0], lo, hi
    return hi[0], lo, hi


E2M1 = [Fr(0), Fr(1, 2), Fr(1), Fr(3, 2), Fr(2), Fr(3), Fr(4), Fr(6)]


def e2m1(q: Fr) -> int:
    """Nearest of the E2M1 magnitudes, ties to the even code, saturating at
    6; the sign bit is set when q < 0 (the printed thresholds: > 0.25,
    >= 0.75, > 1.25, >= 1.75, > 2.5, >= 3.5, > 5)."""
    a = abs(q)
    best = 0
    for c in range(1, 8):
        d, db = abs(a - E2M1[c]), abs(a - E2M1[best])
        if d < db or (d == db and c % 2 == 0):
            best = c
    return best | (8 if q < 0 else 0)


def dec(x: Fr) -> str:
    """Exact decimal expansion of a dyadic rational (finite)."""
    s = "-" if x < 0 else ""
    a = abs(x)
    ip = a.numerator // a.denominator
    fr = a - ip
    digits = ""
    while fr:
        fr *= 10
        d = fr.numerator // fr.denominator
        digits += str(d)
        fr -= d
    return s + str(ip) + ("." + digits if digits else "")


# ---- the blocks -------------------------------------------------------------------
# (name, global scale as binary32 bits, 16 BF16 element bit patterns)
BLOCKS = [
    # prefill workload's global scale; the maximum sits where
    # (gs * amax) * (1/6) rounds to the next E4M3 subnormal
    ("prefill_gs_amax_order", 0x43ACB90F,
     [0x38F9, 0x3880, 0xB8C0, 0x0000, 0x8000, 0x3800, 0xB7E0, 0x3850,
      0x38F8, 0xB8F9, 0x3700, 0x3860, 0xB800, 0x3880, 0x38A0, 0x3810]),
    # tiny workload's global scale; the same order effect in the normal range
    ("tiny_gs_amax_order", 0x44114C1C,
     [0x3F5E, 0x3F00, 0xBF20, 0x3E80, 0x0000, 0xBE00, 0x3F40, 0x3D80,
      0x3F5D, 0xBF5E, 0x3C00, 0x3F10, 0xBF48, 0x3E40, 0x3EC0, 0x8000]),
    # wide_k workload's global scale; 1 / (sf * (1/gs)) puts two elements
    # just below 1.75 and 3.5 where gs / sf and gs * (1/sf) reach them
    ("wide_k_gs_reciprocal_order", 0x42719E34,
     [0x3C98, 0x3BB2, 0x3C32, 0xBBB2, 0xBC32, 0x3B00, 0x3C00, 0x0000,
      0x3A80, 0xBC80, 0x3C40, 0x3B80, 0xBB40, 0x3C10, 0x3BC0, 0x8000]),
    # decode workload's global scale; 1 / (sf / gs) puts an element below
    # 1.75 and one below 3.5 where the printed chain reaches them
    ("decode_gs_reciprocal_order", 0x43C9EA5E,
     [0x3B38, 0x3A55, 0x3AD5, 0xBA55, 0xBAD5, 0x3A00, 0x3B00, 0x0000,
      0x3980, 0xBB00, 0x3B20, 0x3A80, 0xBA40, 0x3B10, 0x3AC0, 0x8000]),
    # a global scale where even gs * amax / 6 (one division) differs
    ("gs_1914_divide_order", 0x44EF46C0,
     [0x3F47, 0x3F00, 0xBF20, 0x3E80, 0x0000, 0xBE00, 0x3F40, 0x3D80,
      0x3F46, 0xBF47, 0x3C00, 0x3F10, 0xBF30, 0x3E40, 0x3EC0, 0x8000]),
]

C6 = rn32(Fr(1, 6))


def quantise(gs: Fr, ys, order: str = "printed"):
    amax = max(abs(y) for y in ys)
    if order == "amax_gs_first":
        s = rn32(rn32(gs * amax) * C6)
    elif order == "divide_by_6":
        s = rn32(gs * amax / 6)
    else:
        s = rn32(gs * rn32(amax * C6))
    sf, _, _ = e4m3_rne_sat(s)
    sfv = e4m3_value(sf)
    if sfv == 0:
        out = Fr(0)
    elif order == "gs_over_sf":
        out = rn32(gs / sfv)
    elif order == "gs_times_rcp_sf":
        out = rn32(gs * rn32(1 / sfv))
    elif order == "rcp_of_sf_over_gs":
        out = rn32(1 / rn32(sfv / gs))
    else:
        out = rn32(1 / rn32(sfv * rn32(1 / gs)))
    codes = [e2m1(rn32(y * out)) for y in ys]
    packed = [codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(8)]
    return sf, packed


def derive(name, gs_bits, y_bits, lines):
    gs = from_f32_bits(gs_bits)
    ys = [bf16(b) for b in y_bits]
    lines.append("")
    lines.append("== block %s" % name)
    lines.append("gs = binary32 0x%08X = %s" % (gs_bits, dec(gs)))
    lines.append("y  = BF16 %s" % " ".join("%04X" % b for b in y_bits))
    amax = max(abs(y) for y in ys)
    lines.append("amax = max|y| = %s" % dec(amax))
    lines.append("c6 = RN32(1/6) = 0x%08X = %s" % (f32_bits(C6), dec(C6)))
    t_exact = amax * C6
    t = rn32(t_exact)
    lines.append("t = RN32(amax * c6): exact %s -> 0x%08X = %s" % (dec(t_exact), f32_bits(t), dec(t)))
    s_exact = gs * t
    s = rn32(s_exact)
    lines.append("s = RN32(gs * t): exact %s -> 0x%08X = %s" % (dec(s_exact), f32_bits(s), dec(s)))
    sf, lo, hi = e4m3_rne_sat(s)
    lines.append("E4M3 neighbours of s: 0x%02X = %s and 0x%02X = %s, midpoint %s -> sf = 0x%02X" % (
        lo[0], dec(lo[1]), hi[0], dec(hi[1]), dec((lo[1] + hi[1]) / 2), sf))
    sfv = e4m3_value(sf)
    rgs = rn32(1 / gs)
    lines.append("rgs = RN32(1/gs) = 0x%08X = %s" % (f32_bits(rgs), dec(rgs)))
    d_exact = sfv * rgs
    d = rn32(d_exact)
    lines.append("d = RN32(sf * rgs): exact %s -> 0x%08X = %s" % (dec(d_exact), f32_bits(d), dec(d)))
    out = rn32(1 / d) if sfv != 0 else Fr(0)
    lines.append("out = RN32(1/d) = 0x%08X = %s" % (f32_bits(out), dec(out)))
    codes = []
    for i, (b, y) in enumerate(zip(y_bits, ys)):
        q_exact = y * out
        q = rn32(q_exact)
        c = e2m1(q)
        codes.append(c)
        lines.append("  y[%2d] = %s: q = RN32(y * out) = %s (exact %s) -> code %X" % (
            i, dec(y), dec(q), dec(q_exact), c))
    packed = [codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(8)]
    assert (sf, packed) == quantise(gs, ys)
    lines.append("RESULT %s gs=%08X y=%s scale=%02X packed=%s" % (
        name, gs_bits, ",".join("%04X" % b for b in y_bits), sf, ",".join("%02X" % p for p in packed)))
    for order in ("amax_gs_first", "divide_by_6", "gs_over_sf", "gs_times_rcp_sf", "rcp_of_sf_over_gs"):
        sf2, p2 = quantise(gs, ys, order)
        if (sf2, p2) != (sf, packed):
            lines.append("  reordered %s would give scale=%02X packed=%s" % (
                order, sf2, ",".join("%02X" % p for p in p2)))


def main():
    lines = [
        "# NVFP4 block quantiser: blocks that pin the order of its FP32 steps.",
        "# Written by tests/golden/derive_nvfp4_step_order.py (exact rational",
        "# arithmetic, every FP32 rounding shown; no numpy, no oracle).",
        "# Steps (vLLM prepare_trtllm_nvfp4, _quantize_nvfp4_global_scale, in the",
        "# page's order; reciprocals IEEE-rounded, E4M3 round-to-nearest-even with",
        "# saturation at 448):",
        "#   t = RN32(amax * RN32(1/6)); s = RN32(gs * t); sf = E4M3(s)",
        "#   d = RN32(sf * RN32(1/gs)); out = sf != 0 ? RN32(1/d) : 0",
        "#   q_i = RN32(y_i * out); code_i = E2M1(q_i) (sign bit when q_i < 0)",
        "#   packed byte m = code[2m] | code[2m+1] << 4",
    ]
    for name, gs_bits, y_bits in BLOCKS:
        derive(name, gs_bits, y_bits, lines)
    with open(os.path.join(HERE, "nvfp4_step_order.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(l for l in lines if l.startswith("RESULT") or "reordered" in l))


if __name__ == "__main__":
    main()
