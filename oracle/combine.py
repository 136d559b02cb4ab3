"""Oracle for the post-expert combine: per-row RMSNorm of each selected expert
output, routing-weight scaling and top-k sum, skipping invalid slots.

Sources:
  [P1] TensorRT-LLM PR #21356, "Add the Muse Spark Open decoder fast paths",
       description, Triton kernel "Post-expert norm and combine" (weight-first
       RMSNorm of each selected expert row, routing weights, top-k sum per
       token; a row behind an invalid slot -- negative or past the end of the
       expert output -- is never read), "Routing" (the pick order fixes the
       summation order) and "Numerics" (round where the composition rounds).
  [P2] TensorRT-LLM PR #21042, "Add the Muse Spark Open model", Description,
       "MoE": the post-expert RMSNorm is applied to each expert's output before
       the weighted top-k sum.

Readings:
  * gain = gain_center + norm_w in FP32 (as in the pre-expert norm), applied
    to the row before a single BF16 rounding of the normalised row;
  * the variance is taken over the expert row itself, eps inside the root;
  * the weighted sum runs in slot order and is rounded once to BF16; a token
    with no valid slot gets +0.0.

Test infrastructure only.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, f64_to_bf16_bits, round_bf16


def combine(expert_out: np.ndarray, slots: np.ndarray, topk_w: np.ndarray,
            norm_w: np.ndarray, gain_center: float, eps: float):
    """expert_out: [R, H] BF16 bits; slots: [T, k] int; topk_w: [T, k] FP32.

    Returns (out BF16 bits [T, H], magnitude float64 [T, H]) where
    magnitude = sum_j |w_j * z_j| over the valid slots, the scale at which the
    rounding of the sum is judged.
    """
    R, H = expert_out.shape
    slots = np.asarray(slots, dtype=np.int64)
    T, k = slots.shape
    w = np.asarray(topk_w, dtype=np.float32).astype(np.float64)
    gain = (np.float32(gain_center) + np.asarray(norm_w, dtype=np.float32)).astype(np.float64)
    e = np.float64(np.float32(eps))
    acc = np.zeros((T, H), dtype=np.float64)
    mag = np.zeros((T, H), dtype=np.float64)
    for j in range(k):
        r = slots[:, j]
        ok = (r >= 0) & (r < R)
        if not ok.any():
            continue
        rows = bf16_bits_to_f64(expert_out[r[ok]])          # only valid rows are read
        ms = np.mean(rows * rows, axis=1, keepdims=True)
        z = round_bf16(rows * gain[None, :] / np.sqrt(ms + e))
        term = w[ok, j][:, None] * z
        acc[ok] += term
        mag[ok] += np.abs(term)
    return f64_to_bf16_bits(acc), mag
