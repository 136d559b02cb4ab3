"""Oracle for the expert FC1 on NVFP4 input (gather grouped GEMM, Relu2 or
SwiGLU, NVFP4 output).

Sources:
  - TensorRT-LLM PR #21842, "CuTe DSL act-fusion GEMMs: key the early
    accumulator release on the loop index", description: the NVFP4 MoE FC1
    is a block-scaled gather grouped GEMM with a fused activation; its Relu2
    FC1 workload is K 1024, N 2688, 512 experts, top-22; its outputs are FP4
    values with their scale factors.
  - the same description names SwiGLU as the gather kernel's other fused
    activation (its compile check builds Relu2 and SwiGLU variants).
  - vLLM API docs, vllm.models.muse_spark.nvidia.ops.prepare_trtllm_nvfp4:
    the NVFP4 format the FC1 reads (E2M1 codes, two per byte, low nibble
    first; linear E4M3 scales per 16 elements; static global scale) and the
    block quantiser its output goes through (`_quantize_nvfp4_global_scale`).
  - lmdeploy PR #4835, MoE gate v2: the dispatch's grouped layout (rows of
    an expert contiguous, in `perm` order, `offsets` per expert).

Readings where the pages leave a step open:
  * a value stands for code * scale / global_scale (how the quantiser made
    it), so the product of an input and a weight value carries
    1 / (gs_x * gs_w[e]);
  * Relu2(v) = max(v, 0)^2, applied to the exact (real-number) FC1 value,
    rounded once to FP32, then quantised with the static output global scale
    gs_y by the same FP32 block steps as the pre-expert quantiser;
  * weights are [E, N, K] (output features by input features), NVFP4 along K,
    one global scale per expert;
  * output row p is grouped position p of the dispatch (flat slot perm[p],
    token perm[p] // k); positions past offsets[E] hold zero codes and zero
    scales;
  * SwiGLU (the page names it but not its weight layout): the expert's
    weights are [E, 2N, K] with the gate projection in rows 0..N-1 and the up
    projection in rows N..2N-1; output column n is silu(gate_n) * up_n with
    silu(g) = g * sigmoid(g), of the exact FC1 values, rounded once to FP32
    and quantised like the Relu2 output.

Test infrastructure only.
"""
from __future__ import annotations

import numpy as np

from .formats import e2m1_decode, e4m3_decode, e2m1_encode, e4m3_encode_satfinite
from .nvfp4 import BLOCK, dequantize, nvfp4_quantize

_F32 = np.float32


def relu2(v: np.ndarray) -> np.ndarray:
    """max(v, 0)^2 (float64)."""
    r = np.maximum(np.asarray(v, dtype=np.float64), 0.0)
    return r * r


def silu(g: np.ndarray) -> np.ndarray:
    """g * sigmoid(g) = g / (1 + exp(-g)) (float64), evaluated through
    exp(-|g|) so that the exponential never overflows."""
    g = np.asarray(g, dtype=np.float64)
    e = np.exp(-np.abs(g))
    return np.where(g >= 0.0, g / (1.0 + e), g * e / (1.0 + e))


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """silu(gate) * up (float64)."""
    return silu(gate) * np.asarray(up, dtype=np.float64)


def fc1_exact(x_packed, x_scales, gs_x, perm, offsets, k, w_packed, w_scales, gs_w):
    """Real-number FC1 values before the activation, [P, N] float64, for the
    grouped rows p < offsets[E] (zeros elsewhere), and the matching sums of
    |products| (for error bounds)."""
    perm = np.asarray(perm)
    offsets = np.asarray(offsets)
    E = len(offsets) - 1
    P = len(perm)
    N = w_packed.shape[1]
    X = dequantize(x_packed, x_scales, gs_x)                    # [T, K]
    acc = np.zeros((P, N), dtype=np.float64)
    mag = np.zeros((P, N), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 <= r0:
            continue
        tok = perm[r0:r1] // k
        We = dequantize(w_packed[e], w_scales[e], np.float32(gs_w[e]))   # [N, K]
        Xe = X[tok]
        acc[r0:r1] = Xe @ We.T
        mag[r0:r1] = np.abs(Xe) @ np.abs(We).T
    return acc, mag


def expert_fc1_nvfp4(x_packed, x_scales, gs_x, perm, offsets, k, w_packed, w_scales, gs_w, gs_y):
    """FC1 with Relu2 on NVFP4 input and weights, NVFP4 output.

    Returns (packed [P, N/2] uint8, scales [P, N/16] uint8), P = len(perm)."""
    acc, _ = fc1_exact(x_packed, x_scales, gs_x, perm, offsets, k, w_packed, w_scales, gs_w)
    y32 = relu2(acc).astype(np.float32)                       # one rounding
    packed, scales = nvfp4_quantize(y32, gs_y)
    used = int(np.asarray(offsets)[-1])
    packed[used:] = 0
    scales[used:] = 0
    return packed, scales


def expert_fc1_swiglu_nvfp4(x_packed, x_scales, gs_x, perm, offsets, k, w_packed, w_scales, gs_w, gs_y):
    """FC1 with SwiGLU on NVFP4 input and weights [E, 2N, K/2] (gate rows
    first, then up rows), NVFP4 output of width N.

    Returns (packed [P, N/2] uint8, scales [P, N/16] uint8), P = len(perm)."""
    acc, _ = fc1_exact(x_packed, x_scales, gs_x, perm, offsets, k, w_packed, w_scales, gs_w)
    N = acc.shape[1] // 2
    y32 = swiglu(acc[:, :N], acc[:, N:]).astype(np.float32)   # one rounding
    packed, scales = nvfp4_quantize(y32, gs_y)
    used = int(np.asarray(offsets)[-1])
    packed[used:] = 0
    scales[used:] = 0
    return packed, scales


def _block_codes(y32_blocks: np.ndarray, gs: np.float32):
    """E4M3 scale bytes and E2M1 codes of FP32 blocks [M, nb, 16] (the
    quantiser's block steps)."""
    amax = np.max(np.abs(y32_blocks), axis=2)
    s = gs * (amax * (_F32(1.0) / _F32(6.0)))
    sf = e4m3_encode_satfinite(s)
    sf_f = e4m3_decode(sf).astype(np.float32)
    d = sf_f * (_F32(1.0) / gs)
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(sf_f != _F32(0.0), _F32(1.0) / d, _F32(0.0)).astype(np.float32)
    codes = e2m1_encode(y32_blocks * out[:, :, None])
    return sf, codes


def fc1_boundary_blocks(x_packed, x_scales, gs_x, perm, offsets, k, w_packed, w_scales, gs_w, gs_y,
                        adds: int | None = None):
    """Output blocks [P, N/16] whose scale or codes an FP32 evaluation may
    legitimately change.

    An evaluation that sums the K exact products in FP32 (in any order, at
    most `adds` = K roundings on the way), then multiplies by an FP32 alpha
    = 1 / (gs_x * gs_w) (two roundings) and squares in FP32 (one rounding),
    lands within
        |dv| <= alpha * (adds * 2^-24 * sum|p| + 4 * 2^-24 * |sum p|)
    of the exact pre-activation value v, and then y within [lo, hi] with
    lo = max(v - dv, 0)^2 (1 - 2^-22), hi = max(v + dv, 0)^2 (1 + 2^-22).
    A block is flagged when its scale at the lower and upper ends of every
    element's interval differs, or when an element's code does."""
    acc, mag = fc1_exact(x_packed, x_scales, gs_x, perm, offsets, k, w_packed, w_scales, gs_w)
    K = x_packed.shape[1] * 2
    adds = K if adds is None else adds
    u = 2.0 ** -24
    dv = adds * u * mag + 4 * u * np.abs(acc)
    lo = (np.maximum(acc - dv, 0.0) ** 2) * (1 - 4 * u)
    hi = (np.maximum(acc + dv, 0.0) ** 2) * (1 + 4 * u)
    P, N = acc.shape
    gs = _F32(gs_y)
    lo32 = np.nextafter(lo.astype(np.float32), np.float32(0)).reshape(P, N // BLOCK, BLOCK)
    hi32 = np.nextafter(hi.astype(np.float32), np.float32(np.inf)).reshape(P, N // BLOCK, BLOCK)
    lo32 = np.maximum(lo32, np.float32(0))
    sf_lo, c_lo = _block_codes(lo32, gs)
    sf_hi, c_hi = _block_codes(hi32, gs)
    near = (sf_lo != sf_hi) | np.any(c_lo != c_hi, axis=2)
    used = int(np.asarray(offsets)[-1])
    near[used:] = False
    return near


# silu's only stationary point: its minimum, at g = -1 - W(1/e) (W the
# principal Lambert W), where silu'(g) = sigmoid(g) (1 + g (1 - sigmoid(g))) = 0.
SILU_ARGMIN = -1.2784645427610738


def _silu_range(lo: np.ndarray, hi: np.ndarray):
    """Smallest and largest silu over each interval [lo, hi] (silu falls
    below SILU_ARGMIN and rises above it)."""
    a, b = silu(lo), silu(hi)
    smin = np.where((lo <= SILU_ARGMIN) & (SILU_ARGMIN <= hi), silu(SILU_ARGMIN), np.minimum(a, b))
    return smin, np.maximum(a, b)


def _codes_at_scale(y32_blocks: np.ndarray, sf: np.ndarray, gs: np.float32):
    """E2M1 codes of FP32 blocks [M, nb, 16] under the given E4M3 scale bytes
    [M, nb] (the quantiser's steps after its scale)."""
    sf_f = e4m3_decode(sf).astype(np.float32)
    d = sf_f * (_F32(1.0) / gs)
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(sf_f != _F32(0.0), _F32(1.0) / d, _F32(0.0)).astype(np.float32)
    return e2m1_encode(y32_blocks * out[:, :, None])


def fc1_swiglu_boundary_blocks(x_packed, x_scales, gs_x, perm, offsets, k, w_packed, w_scales, gs_w,
                               gs_y, adds: int | None = None, rel: float = 2.0 ** -20):
    """Output blocks [P, N/16] of the SwiGLU FC1 whose scale or codes an FP32
    evaluation may legitimately change.

    The gate and up values carry the Relu2 evaluation's bound (FP32 sums of
    the exact products with at most `adds` roundings, then alpha). The FP32
    evaluation of silu(g) * u (an exponential within a few ulp, an addition,
    a reciprocal within 1 ulp and up to three products) is assumed within
    `rel` (16 ulp) of the value it is given, plus |u| * 2^-140 + 2^-148 where the exponential or the result is
    subnormal (an exact zero stays exact). y then lies between the smallest
    and largest silu(g) * u over the gate and up intervals, widened by that
    error. A block is flagged when
    the E4M3 scale at the smallest and the largest possible block maximum
    differ, or when, at the common scale, an element's code at the two ends of
    its interval differs (a sign change included)."""
    acc, mag = fc1_exact(x_packed, x_scales, gs_x, perm, offsets, k, w_packed, w_scales, gs_w)
    K = x_packed.shape[1] * 2
    near = swiglu_boundary_from_values(acc, mag, K if adds is None else adds, gs_y, rel)
    near[int(np.asarray(offsets)[-1]):] = False
    return near


def swiglu_boundary_from_values(acc, mag, adds: int, gs_y, rel: float = 2.0 ** -20):
    """The SwiGLU boundary test on exact FC1 values acc [P, 2N] and their
    sums of |products| mag [P, 2N] (fc1_swiglu_boundary_blocks' steps after
    the GEMM). Returns the flagged blocks [P, N/16]."""
    u = 2.0 ** -24
    dv = adds * u * mag + 4 * u * np.abs(acc)
    N = acc.shape[1] // 2
    g, up = acc[:, :N], acc[:, N:]
    dg, du = dv[:, :N], dv[:, N:]
    smin, smax = _silu_range(g - dg, g + dg)
    ulo, uhi = up - du, up + du
    corners = np.stack([smin * ulo, smin * uhi, smax * ulo, smax * uhi])
    pmin, pmax = corners.min(axis=0), corners.max(axis=0)
    # an exact zero (g = 0 or u = 0 with no error) is computed exactly
    point_zero = (pmin == 0.0) & (pmax == 0.0)
    slack = np.where(point_zero, 0.0, np.maximum(np.abs(ulo), np.abs(uhi)) * 2.0 ** -140 + 2.0 ** -148)
    ylo = pmin - rel * np.abs(pmin) - slack
    yhi = pmax + rel * np.abs(pmax) + slack
    P = acc.shape[0]
    gs = _F32(gs_y)
    # FP32 ends that enclose [ylo, yhi]
    lo32 = ylo.astype(np.float32)
    lo32 = np.where(lo32.astype(np.float64) > ylo, np.nextafter(lo32, np.float32(-np.inf)), lo32)
    hi32 = yhi.astype(np.float32)
    hi32 = np.where(hi32.astype(np.float64) < yhi, np.nextafter(hi32, np.float32(np.inf)), hi32)
    lo32 = lo32.reshape(P, N // BLOCK, BLOCK)
    hi32 = hi32.reshape(P, N // BLOCK, BLOCK)
    # the block maximum lies between the largest smallest-magnitude and the
    # largest largest-magnitude of its elements
    mlo = np.where((lo32 <= 0) & (hi32 >= 0), np.float32(0), np.minimum(np.abs(lo32), np.abs(hi32)))
    mhi = np.maximum(np.abs(lo32), np.abs(hi32))
    sf_lo = e4m3_encode_satfinite(gs * (mlo.max(axis=2) * (_F32(1.0) / _F32(6.0))))
    sf_hi = e4m3_encode_satfinite(gs * (mhi.max(axis=2) * (_F32(1.0) / _F32(6.0))))
    near = sf_lo != sf_hi
    c_lo = _codes_at_scale(lo32, sf_lo, gs)
    c_hi = _codes_at_scale(hi32, sf_lo, gs)
    near |= np.any(c_lo != c_hi, axis=2)
    return near
