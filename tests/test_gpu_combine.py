"""moe_combine against the oracle: within 2 BF16 ulp (at the scale of the
summands), invalid slots never read (NaN guard rows around the expert
output), every workload shape, ragged token counts, full-size sampling."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as wl
from gpu_helpers import DEV, assert_bf16_within, check_combine, dev, host, note, require_gpu

pytestmark = pytest.mark.gpu

m = pytest.importorskip("moe_token_routing_amd")
GUARD = 3   # NaN rows before row 0 and after row R-1


def _with_guards(eo: np.ndarray):
    """Device buffer of R + 2*GUARD rows, NaN guard rows, and the [R,H] view."""
    R, H = eo.shape
    full = np.full((R + 2 * GUARD, H), wl.BF16_NAN, dtype=np.uint16)
    full[GUARD:GUARD + R] = eo
    d = dev(full)
    return d, d[GUARD:GUARD + R]


def _run_and_check(eo, slots, tw, gain, gc, eps, sample=None, what=""):
    require_gpu()
    T, k = slots.shape
    note("combine %s T=%d R=%d H=%d k=%d" % (what, T, eo.shape[0], eo.shape[1], k))
    _, eo_d = _with_guards(eo)
    out = m.combine(eo_d, dev(slots.astype(np.int32)), dev(tw), dev(gain), gc, eps)
    torch.cuda.synchronize()
    got = host(out)
    rows = np.arange(T) if sample is None else sample
    ref, mag = O.combine(eo, slots[rows], tw[rows], gain, gc, eps)
    frac = assert_bf16_within(got[rows], ref, mag, 2.0, "combine " + what)
    assert not np.isnan(O.bf16_bits_to_f64(got[rows])).any()
    return frac


@pytest.mark.parametrize("name,T", [("tiny", None), ("decode", None), ("large_e", 333), ("wide_k", 777)])
def test_combine_workloads(name, T):
    w = wl.WORKLOADS[name]
    T = w.T if T is None else T
    R = T * w.k
    eo = wl.expert_out(w, R)
    slots, invalid_rows = wl.combine_slots(w, T, R)
    eo[invalid_rows] = wl.BF16_NAN
    tw = wl.routing_weights(w, T)
    gain = wl.combine_gain(w)
    frac = _run_and_check(eo, slots, tw, gain, 0.0, w.eps, what=name)
    assert frac > 0.95


def test_combine_prefill_full_size():
    """Full prefill shape (8192 tokens, 65536 rows of 8192) with slots from the
    dispatch of routed ids (5% invalid tokens); rows past the routed count NaN;
    every token checked."""
    w = wl.WORKLOADS["prefill"]
    mask = wl.token_mask(w)
    ids = wl.synthetic_topk_ids(w, mask=mask)
    counts, offsets, perm, dest = O.dispatch(ids, w.E)
    eo = wl.expert_out(w)
    eo[offsets[-1]:] = wl.BF16_NAN
    slots = dest.reshape(w.T, w.k)
    tw = wl.routing_weights(w)
    tw[mask == 0] = 0
    gain = wl.combine_gain(w)
    require_gpu()
    note("combine prefill-full")
    _, eo_d = _with_guards(eo)
    out = m.combine(eo_d, dev(slots.astype(np.int32)), dev(tw), dev(gain), 0.0, w.eps)
    torch.cuda.synchronize()
    frac = check_combine(eo, slots, tw, gain, 0.0, w.eps, host(out), "combine prefill-full")
    print("prefill-full: bit-equal fraction %.4f" % frac)


def test_combine_edge_cases():
    g = np.random.default_rng(40)
    H = 64
    # every slot invalid -> +0.0; out-of-range in both directions; k = 1 and k = 32
    for T, k in [(1, 1), (5, 32), (300, 3)]:
        R = T * k
        eo = wl.f32_to_bf16_bits(g.standard_normal((R, H)).astype(np.float32))
        slots = np.arange(R, dtype=np.int32).reshape(T, k)
        slots[0, :] = -1
        if T > 2:
            slots[1, 0] = R
            slots[2, -1] = -(1 << 30)
            slots[2, 0] = (1 << 31) - 1
        tw = g.uniform(0, 1, (T, k)).astype(np.float32)
        gain = g.uniform(0.5, 1.5, H).astype(np.float32)
        _run_and_check(eo, slots, tw, gain, 0.0, 1e-6, what="edge T=%d k=%d" % (T, k))
    # eps = 0 with power-of-two rows: exact
    T, k = 7, 4
    R = T * k
    rows = g.choice([-1.0, 1.0], (R, H)) * 2.0 ** g.integers(-3, 3, (R, 1))
    eo = wl.f32_to_bf16_bits(rows.astype(np.float32))
    gain = O.round_bf16(g.uniform(0.5, 1.5, H)).astype(np.float32)
    tw = (2.0 ** g.integers(-3, 1, (T, k))).astype(np.float32)
    slots = g.permutation(R).astype(np.int32).reshape(T, k)
    require_gpu()
    note("combine power-of-two exact")
    out = m.combine(dev(eo), dev(slots), dev(tw), dev(gain), 0.0, 0.0)
    ref, _ = O.combine(eo, slots, tw, gain, 0.0, 0.0)
    np.testing.assert_array_equal(host(out), ref)


@pytest.mark.parametrize("H", [8, 24, 256, 768, 1000, 1024, 1032, 4104, 16384])
def test_combine_widths(H):
    """Widths off the power-of-two grid, up to the maximum; 768 and 1000 take
    one wave per token with bounds checks, 1024 one wave per token without."""
    g = np.random.default_rng(H)
    T, k = 37, 5
    R = T * k + 9
    eo = wl.f32_to_bf16_bits((g.standard_normal((R, H)) * 4).astype(np.float32))
    slots = g.integers(-2, R + 2, (T, k)).astype(np.int32)
    tw = g.uniform(0, 0.5, (T, k)).astype(np.float32)
    gain = g.uniform(-1.5, 1.5, H).astype(np.float32)
    _run_and_check(eo, slots, tw, gain, 0.25, 1e-5, what="H=%d" % H)


def test_combine_empty_and_zero_rows():
    require_gpu()
    out = m.combine(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV),
                    torch.full((3, 2), -1, dtype=torch.int32, device=DEV),
                    torch.ones((3, 2), dtype=torch.float32, device=DEV),
                    torch.ones(64, dtype=torch.float32, device=DEV), 0.0, 1e-6)
    assert (host(out) == 0).all()
    out = m.combine(torch.empty((5, 64), dtype=torch.bfloat16, device=DEV),
                    torch.empty((0, 2), dtype=torch.int32, device=DEV),
                    torch.empty((0, 2), dtype=torch.float32, device=DEV),
                    torch.ones(64, dtype=torch.float32, device=DEV), 0.0, 1e-6)
    assert out.shape == (0, 64)


@pytest.mark.parametrize("T,k,H", [(1, 1, 8192), (5, 32, 8192), (3, 7, 16384), (100, 8, 8192), (37, 5, 16384),
                                   (128, 8, 8192), (256, 8, 8192), (300, 8, 8192)])
def test_combine_one_token_per_cu(T, k, H):
    """Batches of no more tokens than CUs at 8192 or 16384 wide rows take one
    1024-thread block per token, or per half or quarter of a row while CUs
    are left over (four parts up to 64 tokens, two up to 128, one above; 300
    tokens: the 256-thread blocks, beside it): token counts off the
    multiples of 8, k off the row groups, a whole token invalid, out-of-range
    slots, and power-of-two rows exact with eps = 0."""
    g = np.random.default_rng(T * k + H)
    R = T * k + 5
    eo = wl.f32_to_bf16_bits((g.standard_normal((R, H)) * 3).astype(np.float32))
    slots = g.permutation(R)[:T * k].astype(np.int32).reshape(T, k)
    slots[0, 0] = -1
    if T > 2:
        slots[1, :] = -1
        slots[2, -1] = R + 3
    tw = g.uniform(0, 1, (T, k)).astype(np.float32)
    gain = g.uniform(-1.5, 1.5, H).astype(np.float32)
    _run_and_check(eo, slots, tw, gain, 0.5, 1e-6, what="one token per CU T=%d k=%d H=%d" % (T, k, H))
    rows = g.choice([-1.0, 1.0], (R, H)) * 2.0 ** g.integers(-3, 3, (R, 1))
    eo = wl.f32_to_bf16_bits(rows.astype(np.float32))
    gain = O.round_bf16(g.uniform(0.5, 1.5, H)).astype(np.float32)
    tw = (2.0 ** g.integers(-3, 1, (T, k))).astype(np.float32)
    note("combine power-of-two exact T=%d k=%d H=%d" % (T, k, H))
    out = m.combine(dev(eo), dev(slots), dev(tw), dev(gain), 0.0, 0.0)
    ref, _ = O.combine(eo, slots, tw, gain, 0.0, 0.0)
    np.testing.assert_array_equal(host(out), ref)
