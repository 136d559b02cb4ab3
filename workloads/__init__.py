"""Seeded synthetic inputs for the MoE routing-and-combine path.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark. It only draws random numbers and stores them in the formats the
path consumes (FP32, BF16 bit patterns, u8 masks, int32 slot tables); it does
none of the method's arithmetic.

Workloads (token count T, hidden width H, experts E, picks per token k):

  tiny      T=16     H=256   E=16    k=4   FP32 hidden N(0,1), router W N(0,0.02),
                                           bias U(-0.1,0.1); combine over [T*k,H]
                                           expert rows with 10% of slots -1 and
                                           their rows NaN-filled
  decode    T=128    H=8192  E=256   k=8   BF16 hidden N(0,1), W N(0,0.01), bias
                                           U(-0.05,0.05); 25% of tokens get
                                           logits on a 2^-8 grid (tie run);
                                           5% invalid combine slots
  prefill   T=8192   H=8192  E=256   k=8   BF16 hidden N(0,1), W N(0,0.01),
                                           bias U(-0.05,0.05); 5% invalid tokens
  large_e   T=4096   H=4096  E=2560  k=8   bias +2.0 on 16 hot experts; 2%
                                           invalid combine slots
  wide_k    T=32768  H=1024  E=512   k=22  BF16 hidden N(0,2) with 1% of the
                                           elements scaled x50; all slots valid

The random streams are numpy PCG64 seeded with 20261203 + the workload's index,
drawn in a fixed order per field (each field gets its own child stream, so a
field can be drawn without drawing the others).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BASE_SEED = 20261203


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    T: int
    H: int
    E: int
    k: int
    hidden_dtype: str  # "f32" or "bf16"
    hidden_std: float
    w_std: float
    bias_lim: float
    hot_experts: int = 0          # experts whose bias is shifted by hot_shift
    hot_shift: float = 0.0
    outlier_frac: float = 0.0     # fraction of hidden elements scaled by outlier_mul
    outlier_mul: float = 1.0
    invalid_token_frac: float = 0.0
    invalid_slot_frac: float = 0.0   # standalone combine: slots made invalid
    tie_token_frac: float = 0.0      # tokens whose logits sit on a 2^-8 grid
    combine_gain_lo: float = 0.5
    combine_gain_hi: float = 1.5
    eps: float = 1e-6
    quant_gain_lim: float = 0.5      # norm weight of the pre-expert norm: U(-lim, lim)
    quant_gain_center: float = 1.0

    @property
    def R(self) -> int:
        """Rows of the expert output: one per routed slot."""
        return self.T * self.k


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 0, 16, 256, 16, 4, "f32", 1.0, 0.02, 0.1,
                 invalid_slot_frac=0.10),
        Workload("decode", 1, 128, 8192, 256, 8, "bf16", 1.0, 0.01, 0.05,
                 invalid_slot_frac=0.05, tie_token_frac=0.25),
        Workload("prefill", 2, 8192, 8192, 256, 8, "bf16", 1.0, 0.01, 0.05,
                 invalid_token_frac=0.05),
        Workload("large_e", 3, 4096, 4096, 2560, 8, "bf16", 1.0, 0.01, 0.05,
                 hot_experts=16, hot_shift=2.0, invalid_slot_frac=0.02),
        Workload("wide_k", 4, 32768, 1024, 512, 22, "bf16", 2.0, 0.02, 0.05,
                 outlier_frac=0.01, outlier_mul=50.0),
    ]
}

# Field order fixes the child stream each field draws from.
_FIELDS = ["hidden", "W", "bias", "mask", "tie_logits", "expert_out", "slots",
           "combine_gain", "quant_x", "quant_gain", "topk_w", "fc1_x", "fc1_w"]

# Output features of the expert FC1 where a workload stands for the FC1 the
# act-fusion GEMM page times (K 1024, N 2688, 512 experts, top-22).
FC1_N = {"wide_k": 2688}
# Output columns of the SwiGLU form of the same FC1: the 2688 weight rows
# split into gate and up halves.
FC1_SWIGLU_N = {"wide_k": 1344}


def rng(workload: Workload, field: str) -> np.random.Generator:
    """Independent PCG64 stream for one field of one workload."""
    seq = np.random.SeedSequence(BASE_SEED + workload.index)
    child = seq.spawn(len(_FIELDS))[_FIELDS.index(field)]
    return np.random.Generator(np.random.PCG64(child))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Store FP32 draws as BF16 bit patterns, rounding to nearest even.

    Only finite draws come through here (NaN fills are written as bit patterns
    directly)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


BF16_NAN = np.uint16(0x7FC0)


def _normal_bf16(g: np.random.Generator, shape, std: float, chunk_rows: int = 4096) -> np.ndarray:
    """N(0, std) draws stored as BF16, generated in row chunks to bound memory."""
    rows = shape[0]
    out = np.empty(shape, dtype=np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        d = g.standard_normal((r1 - r0,) + tuple(shape[1:]), dtype=np.float32)
        if std != 1.0:
            d *= np.float32(std)
        out[r0:r1] = f32_to_bf16_bits(d)
    return out


def hidden(w: Workload, T: Optional[int] = None) -> np.ndarray:
    """Router input [T,H]: FP32 (tiny) or BF16 bits, N(0, hidden_std), with
    optional outliers (a seeded fraction of elements multiplied by outlier_mul
    before the BF16 rounding)."""
    T = w.T if T is None else T
    g = rng(w, "hidden")
    d = g.standard_normal((T, w.H), dtype=np.float32) * np.float32(w.hidden_std)
    if w.outlier_frac > 0:
        n = int(round(w.outlier_frac * T * w.H))
        pos = g.choice(T * w.H, size=n, replace=False)
        d.reshape(-1)[pos] *= np.float32(w.outlier_mul)
    if w.hidden_dtype == "f32":
        return d
    return f32_to_bf16_bits(d)


def router_weight(w: Workload) -> np.ndarray:
    """Router weight [E,H] FP32, N(0, w_std)."""
    return rng(w, "W").standard_normal((w.E, w.H), dtype=np.float32) * np.float32(w.w_std)


def hot_expert_ids(w: Workload) -> np.ndarray:
    if w.hot_experts == 0:
        return np.zeros(0, dtype=np.int64)
    g = rng(w, "bias")
    g.uniform(size=w.E)  # the bias draw comes first on this stream
    return np.sort(g.choice(w.E, size=w.hot_experts, replace=False))


def bias(w: Workload) -> np.ndarray:
    """Selection bias [E] FP32: U(-lim, lim), plus hot_shift on the hot experts."""
    g = rng(w, "bias")
    b = (g.uniform(size=w.E) * 2.0 - 1.0) * w.bias_lim
    b = b.astype(np.float32)
    hot = hot_expert_ids(w)
    b[hot] = (b[hot] + np.float32(w.hot_shift)).astype(np.float32)
    return b


def token_mask(w: Workload, T: Optional[int] = None) -> np.ndarray:
    """Per-token validity [T] u8 (1 valid, 0 invalid); invalid_token_frac of the
    tokens, chosen by a seeded draw, are invalid."""
    T = w.T if T is None else T
    m = np.ones(T, dtype=np.uint8)
    if w.invalid_token_frac > 0:
        n = int(round(w.invalid_token_frac * T))
        m[rng(w, "mask").choice(T, size=n, replace=False)] = 0
    return m


def tie_logits(w: Workload, T: Optional[int] = None) -> np.ndarray:
    """Logits [T,E] FP32 for the logits-in tie run: N(0, sqrt(H)*w_std) (the
    spread of the projection's output), rounded to a 2^-8 grid on
    tie_token_frac of the tokens so that equal keys occur."""
    T = w.T if T is None else T
    g = rng(w, "tie_logits")
    sd = float(np.sqrt(w.H) * w.w_std * w.hidden_std)
    lg = (g.standard_normal((T, w.E)) * sd).astype(np.float32)
    n = int(round(w.tie_token_frac * T))
    rows = g.choice(T, size=n, replace=False) if n else np.zeros(0, dtype=np.int64)
    lg[rows] = (np.round(lg[rows].astype(np.float64) * 256.0) / 256.0).astype(np.float32)
    return lg


def expert_out(w: Workload, R: Optional[int] = None, chunk_rows: int = 4096) -> np.ndarray:
    """Expert output rows [R,H] BF16 bits, N(0,1)."""
    R = w.R if R is None else R
    return _normal_bf16(rng(w, "expert_out"), (R, w.H), 1.0, chunk_rows)


def combine_slots(w: Workload, T: Optional[int] = None, R: Optional[int] = None):
    """Standalone combine slot table [T,k] int32 and the rows it invalidated.

    Slot (t, j) points at expert row t*k + j; invalid_slot_frac of the slots are
    made invalid, half as -1 and half as an index >= R (tiny: all -1). Returns
    (slots, invalid_rows) where invalid_rows are the rows no valid slot reads
    (to be NaN-filled by the caller)."""
    T = w.T if T is None else T
    R = T * w.k if R is None else R
    g = rng(w, "slots")
    slots = np.arange(T * w.k, dtype=np.int64)
    n = int(round(w.invalid_slot_frac * T * w.k))
    bad = g.choice(T * w.k, size=n, replace=False) if n else np.zeros(0, dtype=np.int64)
    if w.name == "tiny":
        slots[bad] = -1
    else:
        half = n // 2
        slots[bad[:half]] = -1
        slots[bad[half:]] = R + g.integers(0, 1 << 20, size=n - half)
    invalid_rows = np.setdiff1d(np.arange(R), slots[(slots >= 0) & (slots < R)])
    return slots.reshape(T, w.k).astype(np.int32), invalid_rows


def combine_gain(w: Workload) -> np.ndarray:
    """Post-expert RMSNorm gain [H] FP32, U(lo, hi) (gain centre 0)."""
    g = rng(w, "combine_gain")
    return (w.combine_gain_lo + g.uniform(size=w.H) * (w.combine_gain_hi - w.combine_gain_lo)).astype(np.float32)


def routing_weights(w: Workload, T: Optional[int] = None) -> np.ndarray:
    """Standalone combine weights [T,k] FP32: U(0.001, 2/k) draws (any
    non-negative weights exercise the combine; these are of the size the
    routing produces)."""
    T = w.T if T is None else T
    u = rng(w, "topk_w").uniform(0.001, 2.0 / w.k, size=(T, w.k))
    return u.astype(np.float32)


def synthetic_topk_ids(w: Workload, T: Optional[int] = None, mask: Optional[np.ndarray] = None) -> np.ndarray:
    """Routing ids [T,k] int32 drawn directly (k distinct experts per token,
    uniformly; hot experts first when the workload has them), -1 for tokens
    whose mask byte is 0. Stands in for a router's output where a test needs
    ids without running one."""
    T = w.T if T is None else T
    g = rng(w, "slots")
    g.integers(0, 2)  # separate this use of the stream from combine_slots
    ids = np.empty((T, w.k), dtype=np.int32)
    hot = hot_expert_ids(w)
    pool = hot if len(hot) >= w.k else np.arange(w.E)
    for t in range(T):
        ids[t] = g.choice(pool, size=w.k, replace=False)
    if mask is not None:
        ids[np.asarray(mask) == 0] = -1
    return ids


def quant_input(w: Workload, T: Optional[int] = None) -> np.ndarray:
    """Pre-expert norm input [T,H] BF16 bits, drawn like the router input
    (hidden_std, outliers) but from its own stream, so it is a distinct buffer."""
    T = w.T if T is None else T
    g = rng(w, "quant_x")
    out = np.empty((T, w.H), dtype=np.uint16)
    for r0 in range(0, T, 4096):
        r1 = min(T, r0 + 4096)
        d = g.standard_normal((r1 - r0, w.H), dtype=np.float32) * np.float32(w.hidden_std)
        if w.outlier_frac > 0:
            n = int(round(w.outlier_frac * d.size))
            pos = g.choice(d.size, size=n, replace=False)
            d.reshape(-1)[pos] *= np.float32(w.outlier_mul)
        out[r0:r1] = f32_to_bf16_bits(d)
    return out


def quant_gain(w: Workload) -> np.ndarray:
    """Pre-expert RMSNorm weight [H] FP32, U(-lim, lim); the gain is
    gain_center + weight."""
    g = rng(w, "quant_gain")
    return ((g.uniform(size=w.H) * 2.0 - 1.0) * w.quant_gain_lim).astype(np.float32)


# E4M3 scale bytes drawn for NVFP4 inputs: exponent fields 6..8, i.e.
# magnitudes 0.5 .. 1.875 * 2 (any byte below 0x7F is a valid scale).
_FC1_SCALE_LO, _FC1_SCALE_HI = 0x30, 0x48


def fc1_activations(w: Workload, T: Optional[int] = None, K: Optional[int] = None):
    """NVFP4 input of the expert FC1 drawn as raw bytes: packed [T, K/2]
    (two uniform E2M1 codes per byte, signs included) and scales [T, K/16]
    (E4M3 bytes); K defaults to the workload's hidden size."""
    T = w.T if T is None else T
    K = w.H if K is None else K
    g = rng(w, "fc1_x")
    packed = g.integers(0, 256, size=(T, K // 2), dtype=np.uint8)
    scales = g.integers(_FC1_SCALE_LO, _FC1_SCALE_HI, size=(T, K // 16), dtype=np.uint8)
    return packed, scales


def fc1_weights(w: Workload, N: int, E: Optional[int] = None, K: Optional[int] = None):
    """NVFP4 FC1 weights drawn as raw bytes: packed [E, N, K/2], scales
    [E, N, K/16] (E4M3 bytes) and one FP32 global scale per expert in
    U(1, 4)."""
    E = w.E if E is None else E
    K = w.H if K is None else K
    g = rng(w, "fc1_w")
    packed = np.empty((E, N, K // 2), dtype=np.uint8)
    for e in range(E):   # per expert, to bound the temporary
        packed[e] = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = g.integers(_FC1_SCALE_LO, _FC1_SCALE_HI, size=(E, N, K // 16), dtype=np.uint8)
    gs = g.uniform(1.0, 4.0, size=E).astype(np.float32)
    return packed, scales, gs
