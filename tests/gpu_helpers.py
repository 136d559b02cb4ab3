"""Shared helpers of the GPU parity tests: host <-> device transfers and the
comparison rules of the parity contract."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle as O

DEV = "cuda:0"


def gpu_available() -> bool:
    return torch.cuda.is_available()


def require_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


def note(msg: str):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    sys.stdout.write("[case] %s\n" % msg)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def scalar_dev(v: float) -> torch.Tensor:
    return torch.tensor([np.float32(v)], dtype=torch.float32, device=DEV)


def assert_bf16_within(got_bits, ref_bits, magnitude, ulps=2.0, what="out"):
    """|got - ref| <= ulps * ulp_bf16(magnitude), elementwise; NaN must match NaN."""
    g = O.bf16_bits_to_f64(got_bits)
    r = O.bf16_bits_to_f64(ref_bits)
    nan_g, nan_r = np.isnan(g), np.isnan(r)
    assert np.array_equal(nan_g, nan_r), "%s: NaN pattern differs" % what
    ok = ~nan_r
    tol = ulps * O.bf16_ulp(np.maximum(np.abs(magnitude), np.abs(r)))
    err = np.abs(g - r)
    bad = ok & (err > tol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d elements beyond %g BF16 ulp, e.g. %s got %s want %s" % (
            what, int(bad.sum()), ulps, idx.tolist(), g[bad][:5], r[bad][:5]))
    return float((g == r)[ok].mean()) if ok.any() else 1.0


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    M = packed.shape[0]
    c = np.empty((M, packed.shape[1] * 2), dtype=np.uint8)
    c[:, 0::2] = packed & 0x0F
    c[:, 1::2] = packed >> 4
    return c


def e2m1_step_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in grid steps between two E2M1 codes (signed values)."""
    va = np.where(a & 8, -1, 1) * (a & 7).astype(np.int64)
    vb = np.where(b & 8, -1, 1) * (b & 7).astype(np.int64)
    # -0 and +0 are one step apart only if a value crossed zero; count index distance
    return np.abs(va - vb)


def check_nvfp4(x, nw, gc, eps, gs, got_packed, got_scales, what="nvfp4", chunk=2048):
    """The NVFP4 parity rule on rows x [M,H] (BF16 bits) and the GPU's packed
    codes / scales for the same rows: codes and scales bit-exact outside the
    stated set of blocks (an element within 2^-19 relative of a BF16 rounding
    midpoint), within one E4M3 / E2M1 step inside it. Row chunks bound the
    oracle's memory. Returns (stated-set blocks, code mismatches inside)."""
    nset = nmis = 0
    for r0 in range(0, x.shape[0], chunk):
        r1 = min(x.shape[0], r0 + chunk)
        ref_packed, ref_scales = O.norm_quant_nvfp4(x[r0:r1], nw, gc, eps, gs)
        near = O.midpoint_boundary_blocks(x[r0:r1], nw, gc, eps)       # [M, H/16]
        gsf = got_scales[r0:r1]
        gc_, rc_ = unpack_codes(got_packed[r0:r1]), unpack_codes(ref_packed)
        nearel = np.repeat(near, 16, axis=1)
        assert np.array_equal(gsf[~near], ref_scales[~near]), what + ": scale mismatch outside the stated set"
        bad = (gc_ != rc_) & ~nearel
        assert not bad.any(), "%s: %d code mismatches outside the stated set" % (what, int(bad.sum()))
        if near.any():
            assert (np.abs(gsf[near].astype(int) - ref_scales[near].astype(int)) <= 1).all(), what
            assert (e2m1_step_distance(gc_[nearel], rc_[nearel]) <= 1).all(), what
        nset += int(near.sum())
        nmis += int(((gc_ != rc_) & nearel).sum())
    return nset, nmis


def check_combine(eo, slots, tw, gain, gc, eps, got, what="combine", chunk=1024):
    """The combine parity rule on every row of got [T,H] (BF16 bits): within
    2 BF16 ulp of the oracle at the scale of the summands, no NaN. Token
    chunks bound the oracle's memory. Returns the bit-equal fraction."""
    T = slots.shape[0]
    eq = n = 0
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        ref, mag = O.combine(eo, slots[t0:t1], tw[t0:t1], gain, gc, eps)
        frac = assert_bf16_within(got[t0:t1], ref, mag, 2.0, what)
        assert not np.isnan(O.bf16_bits_to_f64(got[t0:t1])).any(), what + ": NaN in the output"
        eq += frac * (t1 - t0)
        n += t1 - t0
    return eq / max(n, 1)
