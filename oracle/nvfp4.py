"""Oracle for the pre-expert RMSNorm fused with NVFP4 quantisation.

Source: vLLM API docs, vllm.models.muse_spark.nvidia.ops.prepare_trtllm_nvfp4:
  - module text: the norm matches the model's RMSNorm with one BF16 rounding,
    followed by NVFP4 quantisation with a static global scale and linear
    (unswizzled) block scales;
  - `norm_quant_trtllm_nvfp4`: input [M,H] BF16, norm weight, eps, gain
    centre, global scale tensor; outputs packed [M, H/2] uint8 codes and
    [M, H/16] E4M3 scales; H must be a multiple of the block; M = 0 returns
    at once; the kernel runs without FP contraction;
  - `_quantize_nvfp4_global_scale`: the per-16-element block arithmetic, whose
    steps this module takes in the same order;
  - module text and `norm_quant_trtllm_nvfp4`'s docstring: the input may
    instead be the [tp * M, H / tp] result of a dim-0 all-gather of column
    shards (the rank-block layout), read as the same logical [M, H] rows.
Also TensorRT-LLM PR #21356, "Add the Muse Spark Open decoder fast paths",
description, "Numerics": the norm adds the 1 (gain centre) to the weight in
FP32 and rounds only its result.

Readings where the page leaves a step open:
  * the approximate reciprocals of the printed quantizer are taken as IEEE
    correctly rounded FP32 reciprocals;
  * the FP32 -> E4M3 conversion rounds to nearest even and saturates at 448;
  * the variance is taken over x itself (not over gain * x), eps inside the
    square root.

Test infrastructure only.
"""
from __future__ import annotations

import numpy as np

from .formats import (bf16_bits_to_f64, bf16_ulp, e2m1_encode, e4m3_decode,
                      e4m3_encode_satfinite, round_bf16)

BLOCK = 16
_F32 = np.float32


def gain_f32(norm_w: np.ndarray, gain_center: float) -> np.ndarray:
    """gain = gain_center + w, one FP32 addition per element."""
    return _F32(gain_center) + np.asarray(norm_w, dtype=np.float32)


def rmsnorm_exact(x_bits: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x * gain / sqrt(mean(x^2) + eps) per row, in float64 (before rounding)."""
    x = bf16_bits_to_f64(x_bits)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x * gain.astype(np.float64) / np.sqrt(ms + np.float64(np.float32(eps)))


def rmsnorm_bf16(x_bits: np.ndarray, norm_w: np.ndarray, gain_center: float, eps: float) -> np.ndarray:
    """RMSNorm with a single BF16 rounding of its result (float64 values)."""
    return round_bf16(rmsnorm_exact(x_bits, gain_f32(norm_w, gain_center), eps))


def nvfp4_quantize(y: np.ndarray, global_scale: float):
    """NVFP4 quantisation of [M, H] values y (BF16 values, exact in FP32).

    Per block of 16 consecutive elements of a row:
      amax  = max |y|
      sf    = E4M3( gs * (amax * (1/6)) )           every product FP32-rounded
      out   = 1 / (f32(sf) * (1/gs))  if sf != 0, else 0
      q     = y * out                                FP32
      code  = E2M1(q), sign bit when q < 0
    and two codes share a byte: the even element in the low nibble.
    Returns (packed uint8 [M, H/2], scales uint8 [M, H/16]).
    """
    y32 = np.asarray(y, dtype=np.float32)
    M, H = y32.shape
    if H % BLOCK:
        raise ValueError("H must be a multiple of 16")
    gs = _F32(global_scale)
    blocks = y32.reshape(M, H // BLOCK, BLOCK)
    amax = np.max(np.abs(blocks), axis=2)
    t = amax * (_F32(1.0) / _F32(6.0))
    s = gs * t
    sf = e4m3_encode_satfinite(s)
    sf_f = e4m3_decode(sf).astype(np.float32)
    d = sf_f * (_F32(1.0) / gs)
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(sf_f != _F32(0.0), _F32(1.0) / d, _F32(0.0)).astype(np.float32)
    q = blocks * out[:, :, None]
    codes = e2m1_encode(q).reshape(M, H)
    packed = (codes[:, 0::2] & np.uint8(0x0F)) | (codes[:, 1::2] << np.uint8(4))
    return packed.astype(np.uint8), sf.astype(np.uint8)


def norm_quant_nvfp4(x_bits, norm_w, gain_center, eps, global_scale):
    """RMSNorm (one BF16 rounding) followed by NVFP4 quantisation."""
    y = rmsnorm_bf16(x_bits, norm_w, gain_center, eps)
    return nvfp4_quantize(y, global_scale)


def rank_block_rows(pooled: np.ndarray, num_tokens: int, hidden: int) -> np.ndarray:
    """The logical [M, H] rows of a rank-block input [tp * M, H / tp]: block r
    (rows r*M .. r*M + M - 1) holds columns r*S .. r*S + S - 1 of every row,
    S = H / tp (prepare_trtllm_nvfp4, `norm_quant_trtllm_nvfp4`). tp = 1 is the
    contiguous layout."""
    pooled = np.asarray(pooled)
    M, S = int(num_tokens), pooled.shape[1]
    assert pooled.shape[0] * S == M * hidden and hidden % S == 0
    tp = hidden // S
    return pooled.reshape(tp, M, S).transpose(1, 0, 2).reshape(M, hidden)


def norm_quant_nvfp4_rank_block(pooled_bits, num_tokens, norm_w, gain_center, eps, global_scale):
    """norm_quant_nvfp4 of the logical rows of a rank-block input."""
    x = rank_block_rows(pooled_bits, num_tokens, np.asarray(norm_w).shape[0])
    return norm_quant_nvfp4(x, norm_w, gain_center, eps, global_scale)


def global_scale(y: np.ndarray) -> np.float32:
    """Static global scale 448 * 6 / amax over the whole normalised tensor
    (FP32 division), so the largest block scale lands on E4M3's maximum."""
    amax = _F32(np.max(np.abs(np.asarray(y, dtype=np.float32))))
    return _F32(2688.0) / amax


def midpoint_boundary_blocks(x_bits, norm_w, gain_center, eps, rel: float = 2.0 ** -19):
    """Blocks [M, H/16] holding an element whose exact normalised value lies
    within a relative distance `rel` of a BF16 rounding midpoint.

    An implementation that evaluates the norm in FP32 carries a relative error
    of about 2^-20 before its BF16 rounding, so near a midpoint it may round
    the other way; that changes the element and possibly the block's amax,
    scale and every code of the block. Outside these blocks the codes and
    scales are fixed exactly by the definition.
    """
    v = rmsnorm_exact(x_bits, gain_f32(norm_w, gain_center), eps)
    u = bf16_ulp(v)
    frac = np.abs(v) / u
    dist = np.abs(frac - np.floor(frac) - 0.5) * u
    near = dist <= rel * np.abs(v)
    M, H = near.shape
    return near.reshape(M, H // BLOCK, BLOCK).any(axis=2)


def dequantize(packed: np.ndarray, scales: np.ndarray, global_scale: float) -> np.ndarray:
    """Values the codes stand for: E2M1 value * E4M3 scale / gs (float64)."""
    from .formats import e2m1_decode
    M = packed.shape[0]
    lo = packed & np.uint8(0x0F)
    hi = packed >> np.uint8(4)
    codes = np.empty((M, packed.shape[1] * 2), dtype=np.uint8)
    codes[:, 0::2] = lo
    codes[:, 1::2] = hi
    v = e2m1_decode(codes).reshape(M, -1, BLOCK)
    sc = e4m3_decode(scales)[:, :, None] / np.float64(np.float32(global_scale))
    return (v * sc).reshape(M, -1)
