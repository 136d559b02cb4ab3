"""Oracle for the expert FC1 on NVFP4 input (gather grouped GEMM, Relu2,
NVFP4 output).

Sources:
  - TensorRT-LLM PR #21842, "CuTe DSL act-fusion GEMMs: key the early
    accumulator release on the loop index", description: the NVFP4 MoE FC1
    is a block-scaled gather grouped GEMM with a fused activation; its Relu2
    FC1 workload is K 1024, N 2688, 512 experts, top-22; its outputs are FP4
    values with their scale factors.
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
    scales.

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
