"""Oracle for the router: projection, sigmoid + bias, sorted top-k with
lowest-id ties, renormalised weights, per-token validity mask.

Sources (each function names the passage it follows):
  [P1] TensorRT-LLM PR #21356, "Add the Muse Spark Open decoder fast paths",
       description, list of Triton kernels: items "Routing" and "Router
       projection"; section "Not in this PR" (BF16x3 router experiment).
  [P2] TensorRT-LLM PR #21042, "Add the Muse Spark Open model", Description,
       paragraph "MoE" (the router runs in FP32).
  [P5] lmdeploy PR #4835, "Intern-S2-Mobius meta-MoE support, MoE gate v2, CP
       attention fixes": commit notes on the per-token validity mask, and the
       Summary's "MoE gate v2 + invalid-token routing" (aux-loss-free gate
       `invokeMoeGate_NoAuxTC`).

Test infrastructure only (tests/, the smoke check, the benchmark's CPU
baseline).
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64


def hidden_to_f64(hidden: np.ndarray) -> np.ndarray:
    """Router input as exact float64: FP32 arrays as they are, uint16 arrays
    as BF16 bit patterns."""
    if hidden.dtype == np.uint16:
        return bf16_bits_to_f64(hidden)
    if hidden.dtype == np.float32:
        return hidden.astype(np.float64)
    raise TypeError("router input must be float32 or BF16 bits (uint16)")


def router_logits(hidden: np.ndarray, W: np.ndarray, scale: float = 1.0):
    """Router projection [P1 "Router projection"; P2 "MoE"].

    logit[t, e] = scale * sum_i h[t, i] * W[e, i], with FP32 weights and the
    input cast to FP32. The oracle forms every product exactly and sums in
    float64 (a float64 matrix product), applies the scale (the pages'
    "metap scale"; its value is an argument) and rounds once to FP32.

    Returns (logits float32 [T,E], magnitude float64 [T,E]) where magnitude =
    |scale| * sum_i |h[t,i] * W[e,i]| bounds the rounding error any FP32
    accumulation order can make.
    """
    h = hidden_to_f64(hidden)
    w = np.asarray(W, dtype=np.float32).astype(np.float64)
    s = np.float64(np.float32(scale))
    dot = h @ w.T
    logits = (s * dot).astype(np.float32)
    magnitude = abs(s) * (np.abs(h) @ np.abs(w).T)
    return logits, magnitude


def sigmoid_f32(logits: np.ndarray) -> np.ndarray:
    """sigmoid(l) = 1 / (1 + exp(-l)) evaluated in float64 and rounded once to
    FP32 [P1 "Routing": sigmoid of the router output]."""
    l64 = np.asarray(logits, dtype=np.float32).astype(np.float64)
    with np.errstate(over="ignore"):
        return (1.0 / (1.0 + np.exp(-l64))).astype(np.float32)


def selection_keys(logits: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """key[t, e] = sigmoid(logit[t, e]) + bias[e], an FP32 addition.

    The bias steers which experts are picked and nothing else [P1 "Routing":
    sigmoid, then bias, then top-k; P5: the aux-loss-free gate]."""
    s = sigmoid_f32(logits)
    return s + np.asarray(bias, dtype=np.float32)[None, :]


def topk_sorted(keys: np.ndarray, k: int) -> np.ndarray:
    """Per row, the k experts with the largest keys, ordered by key from the
    largest down; equal keys are ordered by ascending expert id, so the lowest
    id wins a tie [P1 "Routing": sorted picks, exact ties to the lowest id].

    Equality is IEEE equality (+0 == -0). A NaN key ranks below every number.
    """
    T, E = keys.shape
    ids = np.broadcast_to(np.arange(E), (T, E))
    k64 = keys.astype(np.float64)
    neg = np.where(np.isnan(k64), np.inf, -k64)      # NaN sorts after -inf keys
    nan_last = np.isnan(k64).astype(np.int8)
    neg = np.where(neg == 0.0, 0.0, neg)             # -0.0 and +0.0 compare equal
    # lexsort: last key is primary -> (nan flag, -key, id)
    order = np.lexsort((ids, neg, nan_last), axis=1)
    return order[:, :k].astype(np.int32)


def renormalized_weights(sig: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """w_j = s_{id_j} / (s_{id_0} + ... + s_{id_{k-1}}) with the unbiased
    sigmoid s [P1 "Routing": renormalised weights].

    The denominator is an FP32 running sum in pick order; each weight is one
    correctly rounded FP32 division."""
    T, k = ids.shape
    picked = np.take_along_axis(sig, ids.astype(np.int64), axis=1).astype(np.float32)
    total = np.zeros(T, dtype=np.float32)
    for j in range(k):
        total = total + picked[:, j]
    return picked / total[:, None]


def route_from_logits(logits: np.ndarray, bias: np.ndarray, token_mask: np.ndarray, k: int):
    """Routing of each token from its FP32 logits.

    Valid tokens: ids = top-k of the keys (see topk_sorted), weights =
    renormalized_weights. Invalid tokens (mask byte 0) produce no routing entry:
    ids -1 and weights 0.0, and their logits are never inspected [P5: invalid
    tokens produce no routing entries]. Returns (ids int32 [T,k], w float32 [T,k]).
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    valid = np.asarray(token_mask).astype(bool)
    ids = np.full((T, k), -1, dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float32)
    if valid.any():
        lg = logits[valid]
        keys = selection_keys(lg, bias)
        vid = topk_sorted(keys, k)
        ids[valid] = vid
        w[valid] = renormalized_weights(sigmoid_f32(lg), vid)
    return ids, w


def route(hidden, W, bias, token_mask, k, scale=1.0):
    """Projection followed by routing: returns (logits, magnitude, ids, w)."""
    logits, magnitude = router_logits(hidden, W, scale)
    ids, w = route_from_logits(logits, bias, token_mask, k)
    return logits, magnitude, ids, w


def key_gap_near_ties(logits, magnitude_bound, bias, token_mask, k):
    """Tokens whose routing may legitimately differ when the logits carry an
    error of at most magnitude_bound[t, e].

    A key moves by at most 0.25 * |dlogit| (the sigmoid's slope is <= 1/4) plus
    two FP32 roundings. A token is listed when two adjacent keys among its
    k + 1 largest are closer than the sum of their possible movements, since
    then the pick set or its order can flip. Returns a bool [T] array.
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    keys = selection_keys(logits, bias).astype(np.float64)
    kk = min(k + 1, E)
    order = topk_sorted(keys.astype(np.float32), kk)
    top = np.take_along_axis(keys, order.astype(np.int64), axis=1)
    move = 0.25 * np.take_along_axis(np.asarray(magnitude_bound, np.float64), order.astype(np.int64), axis=1)
    move += 2.0 ** -23 * (np.abs(top) + 1.0)
    gaps = top[:, :-1] - top[:, 1:]
    near = (gaps <= move[:, :-1] + move[:, 1:]).any(axis=1)
    return near & np.asarray(token_mask).astype(bool)
