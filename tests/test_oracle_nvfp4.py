"""Pins of the RMSNorm + NVFP4 oracle: power-of-two rows that make the norm
exact, the printed code thresholds reached through the public function,
scale saturation and underflow, the quantisation error bound, and the
variance taken over x rather than gain * x; the rank-block input layout
rebuilt from the column shards and dim-0 gather that define it."""
import os

import numpy as np
import pytest

import oracle as O
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(v):
    return wl.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def test_power_of_two_rows_make_the_norm_exact():
    g = np.random.default_rng(20)
    H = 64
    for m in (-3, 0, 5):
        signs = g.choice([-1.0, 1.0], size=(3, H))
        x = _bits(signs * 2.0 ** m)
        w = O.round_bf16(g.uniform(-0.5, 0.5, H)).astype(np.float32)   # gain 1 + w exact in BF16? not needed
        gain = O.gain_f32(w, 1.0)
        y = O.rmsnorm_bf16(x, w, 1.0, 0.0)
        np.testing.assert_array_equal(y, O.round_bf16(signs * gain.astype(np.float64)))


def test_constant_row_ignores_the_gain_in_the_variance():
    # variance over x: a constant row normalises to sign(c) * gain exactly
    H = 32
    gain = np.linspace(0.25, 2.0, H).astype(np.float32)
    for c in (0.375, -3.0, 1e-3):
        x = _bits(np.full((1, H), c))
        y = O.rmsnorm_bf16(x, gain, 0.0, 0.0)
        np.testing.assert_array_equal(y[0], O.round_bf16(np.sign(c) * gain.astype(np.float64)))


def _threshold_rows():
    vals, codes = [], []
    with open(os.path.join(GOLDEN, "e2m1_thresholds.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            v, c = line.split()
            val = float.fromhex(v) if v.startswith("0x") else float(v)
            if np.isfinite(val) and val <= 6.0 and O.round_bf16(np.array([val]))[0] == val:
                vals.append(val)
                codes.append(int(c))
    return np.array(vals), np.array(codes, dtype=np.uint8)


def test_printed_thresholds_through_norm_and_quant():
    # Rows of +-1 with eps = 0 normalise to exactly +-gain. Each block holds a
    # 6 (its amax) so that, with global scale 1, the block scale is exactly 1
    # and the codes are the E2M1 codes of the gains themselves.
    vals, want = _threshold_rows()
    n = len(vals)
    per_block = 15
    nb = -(-n // per_block)
    H = nb * 16
    gain = np.zeros(H, dtype=np.float32)
    expect = np.zeros(H, dtype=np.uint8)
    for b in range(nb):
        gain[b * 16] = 6.0
        expect[b * 16] = 7
        chunk = vals[b * per_block:(b + 1) * per_block]
        gain[b * 16 + 1: b * 16 + 1 + len(chunk)] = chunk
        expect[b * 16 + 1: b * 16 + 1 + len(chunk)] = want[b * per_block:(b + 1) * per_block]
    for sgn in (1.0, -1.0):
        x = _bits(np.full((1, H), sgn))
        packed, sf = O.norm_quant_nvfp4(x, gain, 0.0, 0.0, 1.0)
        assert (sf == 0x38).all()                               # scale 1.0
        codes = np.empty(H, dtype=np.uint8)
        codes[0::2] = packed[0] & 0xF
        codes[1::2] = packed[0] >> 4
        exp = expect | (np.uint8(8) if sgn < 0 else np.uint8(0))
        exp = np.where((sgn < 0) & (gain == 0), np.uint8(0), exp)   # -1 * 0 = -0.0: no sign bit
        np.testing.assert_array_equal(codes, exp)


def test_scale_saturation_underflow_and_zero_blocks():
    g = np.random.default_rng(21)
    x = _bits(g.standard_normal((4, 64)))
    w = np.zeros(64, np.float32)
    _, sf = O.norm_quant_nvfp4(x, w, 1.0, 1e-6, 1e9)
    assert (sf == 0x7E).all()
    packed, sf = O.norm_quant_nvfp4(x, w, 1.0, 1e-6, 1e-9)
    assert (sf == 0).all() and (packed == 0).all()
    z = np.zeros((2, 32), np.uint16)
    packed, sf = O.norm_quant_nvfp4(z, w[:32], 1.0, 1e-6, 100.0)
    assert (sf == 0).all() and (packed == 0).all()


@pytest.mark.parametrize("name", ["tiny", "wide_k"])
def test_quantisation_error_bound_and_global_scale(name):
    w_ = wl.WORKLOADS[name]
    T = 64
    x = wl.quant_input(w_, T)
    nw = wl.quant_gain(w_)
    y = O.rmsnorm_bf16(x, nw, w_.quant_gain_center, w_.eps)
    gs = O.global_scale(y)
    packed, sf = O.nvfp4_quantize(y, gs)
    # the block holding the tensor's amax gets the largest scale, 448
    b = np.unravel_index(np.argmax(np.abs(y)), y.shape)
    assert sf[b[0], b[1] // 16] == 0x7E
    assert sf.max() == 0x7E
    # each block scale is the E4M3 rounding of gs * amax / 6 (<= 2^-4 relative
    # half step, or the subnormal half step 2^-10)
    amax = np.abs(y).reshape(T, -1, 16).max(2)
    target = np.float64(gs) * amax / 6
    sv = O.e4m3_decode(sf)
    assert (np.abs(sv - target) <= np.maximum(target * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6)).all()
    # every element is within half an E2M1 step (at its magnitude) of its code's value
    dq = O.dequantize(packed, sf, gs)
    unit = (sv / np.float64(gs))[:, :, None]             # the value code 1.0 stands for
    q = (y.reshape(T, -1, 16) / np.where(unit == 0, 1, unit))
    half = np.where(np.abs(q) < 2, 0.25, np.where(np.abs(q) < 4, 0.5, 1.0))
    err = np.abs(dq.reshape(T, -1, 16) - y.reshape(T, -1, 16))
    bound = half * unit * (1 + 2.0 ** -20) + np.maximum(np.abs(q) - 6, 0) * unit
    assert (err <= bound + 1e-30).all()


def test_boundary_blocks_flag_midpoints():
    H = 32
    gain = np.ones(H, np.float32)
    x = _bits(np.ones((1, H)))
    gain2 = gain.copy()
    gain2[3] = np.float32(1.0 + 2 ** -8)          # exactly a BF16 midpoint after the norm
    near = O.midpoint_boundary_blocks(x, gain2, 0.0, 0.0)
    np.testing.assert_array_equal(near, [[True, False]])
    near = O.midpoint_boundary_blocks(x, gain, 0.0, 0.0)
    assert not near.any()


@pytest.mark.parametrize("tp", [1, 2, 4, 8])
def test_rank_block_layout_is_the_gathered_column_shards(tp):
    """The rank-block input is what a dim-0 all-gather of column shards
    leaves (prepare_trtllm_nvfp4, `norm_quant_trtllm_nvfp4`): build it that
    way -- each rank keeps columns [r*S, (r+1)*S) of every row, the ranks'
    pieces are stacked along dim 0 -- and read it back, both through the
    oracle and element by element by the stacking rule."""
    M, H = 5, 128
    g = np.random.default_rng(40 + tp)
    x = g.integers(0, 1 << 16, size=(M, H), dtype=np.uint16)
    S = H // tp
    pooled = np.concatenate([x[:, r * S:(r + 1) * S] for r in range(tp)], axis=0)
    assert pooled.shape == (tp * M, S)
    assert np.array_equal(O.rank_block_rows(pooled, M, H), x)
    for t in range(M):
        for i in range(H):
            assert pooled[(i // S) * M + t, i % S] == x[t, i]


def test_rank_block_quant_matches_contiguous():
    w = wl.WORKLOADS["wide_k"]
    M, H = 9, w.H
    x = wl.quant_input(w, M)
    nw = wl.quant_gain(w)
    gs = np.float32(3.0)
    ref = O.norm_quant_nvfp4(x, nw, w.quant_gain_center, w.eps, gs)
    for tp in (2, 8):
        S = H // tp
        pooled = np.concatenate([x[:, r * S:(r + 1) * S] for r in range(tp)], axis=0)
        got = O.norm_quant_nvfp4_rank_block(pooled, M, nw, w.quant_gain_center, w.eps, gs)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def _step_order_blocks():
    """The RESULT lines of golden/nvfp4_step_order.txt: hand-checkable blocks
    (every FP32 rounding written out in exact arithmetic) whose scale byte or
    codes depend on the order of the quantiser's steps (vLLM
    prepare_trtllm_nvfp4, _quantize_nvfp4_global_scale)."""
    out = []
    with open(os.path.join(GOLDEN, "nvfp4_step_order.txt")) as f:
        for line in f:
            if not line.startswith("RESULT "):
                continue
            fields = dict(kv.split("=") for kv in line.split()[2:])
            gs = np.array([int(fields["gs"], 16)], np.uint32).view(np.float32)[0]
            y = np.array([int(b, 16) for b in fields["y"].split(",")], np.uint16)
            scale = int(fields["scale"], 16)
            packed = np.array([int(b, 16) for b in fields["packed"].split(",")], np.uint8)
            out.append((line.split()[1], gs, y, scale, packed))
    return out


def test_step_order_golden_blocks():
    blocks = _step_order_blocks()
    assert len(blocks) == 5
    for name, gs, y, scale, packed in blocks:
        yv = O.bf16_bits_to_f64(y).astype(np.float32)[None, :]
        p, s = O.nvfp4_quantize(yv, gs)
        assert int(s[0, 0]) == scale, name
        np.testing.assert_array_equal(p[0], packed, err_msg=name)


def _reordered_quantize(y, gs, order):
    """A deliberately reordered quantiser (numpy FP32), to show that the
    golden blocks tell the printed order from its plausible rearrangements."""
    F = np.float32
    y = np.asarray(y, np.float32)
    amax = np.max(np.abs(y))
    if order == "gs_amax_first":
        s = (F(gs) * amax) * (F(1) / F(6))
    else:
        s = F(gs) * (amax * (F(1) / F(6)))
    sf = O.e4m3_encode_satfinite(np.array([s], np.float32))
    sfv = O.e4m3_decode(sf).astype(np.float32)[0]
    if sfv == 0:
        out = F(0)
    elif order == "gs_over_sf":
        out = F(gs) / sfv
    elif order == "rcp_of_sf_over_gs":
        out = F(1) / (sfv / F(gs))
    else:
        out = F(1) / (sfv * (F(1) / F(gs)))
    codes = O.e2m1_encode(y * out)
    return codes[0::2] | (codes[1::2] << 4), int(sf[0])


@pytest.mark.parametrize("order", ["gs_amax_first", "gs_over_sf", "rcp_of_sf_over_gs"])
def test_step_order_golden_rejects_reordered_chains(order):
    blocks = _step_order_blocks()
    printed_ok = all(
        (lambda r: r[1] == scale and np.array_equal(r[0], packed))(
            _reordered_quantize(O.bf16_bits_to_f64(y), gs, "printed"))
        for _, gs, y, scale, packed in blocks)
    assert printed_ok
    mismatched = [name for name, gs, y, scale, packed in blocks
                  if (lambda r: r[1] != scale or not np.array_equal(r[0], packed))(
                      _reordered_quantize(O.bf16_bits_to_f64(y), gs, order))]
    assert mismatched, order + " passes every golden block"
