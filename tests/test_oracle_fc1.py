"""Pins of the expert FC1 oracle (NVFP4 gather grouped GEMM + Relu2 + NVFP4
output): a written-out loop over (row, column, k) with table decoding of the
formats, a one-hot case whose values, scale and codes follow by hand, the
boundary set on a value placed exactly on a printed code threshold, and the
error bound of the quantised output."""
import numpy as np
import pytest

import oracle as O
import workloads as wl

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _e4m3(c):
    c = int(c)
    e, m = (c >> 3) & 15, c & 7
    v = m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10)
    return -v if c & 0x80 else v


def _code_value(byte, half):
    c = (int(byte) >> (4 * half)) & 15
    v = E2M1[c & 7]
    return -v if c & 8 else v


def _decode(packed_row, scale_row, gs, i):
    return _code_value(packed_row[i // 2], i % 2) * _e4m3(scale_row[i // 16]) / float(np.float32(gs))


def _small_case(seed, T=5, k=3, E=4, K=32, N=32):
    g = np.random.default_rng(seed)
    xp = g.integers(0, 256, size=(T, K // 2), dtype=np.uint8)
    xs = g.integers(0x30, 0x41, size=(T, K // 16), dtype=np.uint8)
    wp = g.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    ws = g.integers(0x30, 0x41, size=(E, N, K // 16), dtype=np.uint8)
    ids = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[1, 2] = -1                                           # one invalid slot
    perm, dest, offsets = _grouped(ids, E)
    return xp, xs, np.float32(3.0), perm, offsets, k, wp, ws, np.linspace(1.5, 4.0, E).astype(np.float32)


def _grouped(ids, E):
    counts, offsets, perm, dest = O.dispatch(ids, E)
    return perm, dest, offsets


def test_fc1_matches_a_written_out_loop():
    xp, xs, gx, perm, offsets, k, wp, ws, gw = _small_case(3)
    acc, mag = O.fc1_exact(xp, xs, gx, perm, offsets, k, wp, ws, gw)
    K, N = xp.shape[1] * 2, wp.shape[1]
    E = len(offsets) - 1
    for p in range(len(perm)):
        if p >= offsets[-1]:
            assert not acc[p].any()
            continue
        e = max(i for i in range(E) if offsets[i] <= p)
        t = perm[p] // k
        for n in range(N):
            s = sum(_decode(xp[t], xs[t], gx, i) * _decode(wp[e, n], ws[e, n], gw[e], i) for i in range(K))
            m = sum(abs(_decode(xp[t], xs[t], gx, i) * _decode(wp[e, n], ws[e, n], gw[e], i)) for i in range(K))
            assert acc[p, n] == pytest.approx(s, rel=1e-12, abs=1e-12)
            assert mag[p, n] == pytest.approx(m, rel=1e-12, abs=1e-12)


def test_fc1_one_hot_values_scale_and_codes():
    """K = 16, the input one-hot at k = 0 with value 1: the FC1 value of output
    column n is the weight w[n, 0]. Weight 2.5 (code 2.0 x scale 1.25) gives
    Relu2 6.25, the block maximum: 6.25 * RN32(1/6) rounds to E4M3 1.0, so the
    output scale is 1 and q = y: 6.25 saturates to code 7, 0.25 sits on the
    printed threshold (> 0.25 is needed for code 1) and gives code 0, 1.0 is
    code 2, and a negative weight gives 0."""
    K, N = 16, 16
    xp = np.zeros((1, K // 2), dtype=np.uint8)
    xp[0, 0] = 0x02                                          # element 0 = 1.0, element 1 = 0
    xs = np.array([[0x38]], dtype=np.uint8)                  # scale 1.0
    wp = np.zeros((1, N, K // 2), dtype=np.uint8)
    ws = np.full((1, N, 1), 0x38, dtype=np.uint8)
    wp[0, 0, 0], ws[0, 0, 0] = 0x04, 0x3A                    # 2.0 * 1.25 = 2.5
    wp[0, 1, 0] = 0x01                                       # 0.5
    wp[0, 2, 0] = 0x02                                       # 1.0
    wp[0, 3, 0] = 0x0C                                       # -2.0
    perm = np.array([0], dtype=np.int32)
    offsets = np.array([0, 1], dtype=np.int32)
    acc, _ = O.fc1_exact(xp, xs, 1.0, perm, offsets, 1, wp, ws, np.array([1.0], np.float32))
    assert list(acc[0, :4]) == [2.5, 0.5, 1.0, -2.0]
    packed, scales = O.expert_fc1_nvfp4(xp, xs, 1.0, perm, offsets, 1, wp, ws, np.array([1.0], np.float32), 1.0)
    assert scales[0, 0] == 0x38
    codes = [(packed[0, i // 2] >> (4 * (i % 2))) & 15 for i in range(N)]
    assert codes[:5] == [7, 0, 2, 0, 0]
    near = O.fc1_boundary_blocks(xp, xs, 1.0, perm, offsets, 1, wp, ws, np.array([1.0], np.float32), 1.0)
    assert near[0, 0]                                        # 0.25 is on a threshold
    wp[0, 1, 0] = 0x02
    ws[0, 1, 0] = 0x36                                       # 1.0 * 0.75: Relu2 0.5625, code 1, far from 0.25 / 0.75
    near = O.fc1_boundary_blocks(xp, xs, 1.0, perm, offsets, 1, wp, ws, np.array([1.0], np.float32), 1.0)
    assert not near[0, 0]


def test_fc1_unused_positions_are_zero_and_rows_follow_their_slot():
    xp, xs, gx, perm, offsets, k, wp, ws, gw = _small_case(5)
    acc, _ = O.fc1_exact(xp, xs, gx, perm, offsets, k, wp, ws, gw)
    y = O.relu2(acc)
    gy = O.global_scale(y)
    packed, scales = O.expert_fc1_nvfp4(xp, xs, gx, perm, offsets, k, wp, ws, gw, gy)
    used = int(offsets[-1])
    assert used == len(perm) - 1                             # one invalid slot
    assert not packed[used:].any() and not scales[used:].any()
    # the same (token, expert) pair in two tokens' slots gives the same row
    ids = np.array([[0, 1], [1, 0]], dtype=np.int32)
    perm2, _, off2 = _grouped(ids, 2)
    xp2 = np.repeat(xp[:1], 2, axis=0)
    xs2 = np.repeat(xs[:1], 2, axis=0)
    a2, _ = O.fc1_exact(xp2, xs2, gx, perm2, off2, 2, wp[:2], ws[:2], gw[:2])
    assert np.array_equal(a2[0], a2[1]) and np.array_equal(a2[2], a2[3])


def test_fc1_quantised_output_within_the_block_error_bound():
    """The dequantised output is Relu2 of the exact value within half a code
    step of the block's scale (plus the scale's own rounding): NVFP4's
    worst case is |err| <= (1/2 of the local E2M1 step) * scale / gs_y, and
    never more than a quarter of the block maximum."""
    xp, xs, gx, perm, offsets, k, wp, ws, gw = _small_case(9, T=8, k=4, E=6, K=64, N=48)
    acc, _ = O.fc1_exact(xp, xs, gx, perm, offsets, k, wp, ws, gw)
    y = O.relu2(acc)
    gy = O.global_scale(y)
    packed, scales = O.expert_fc1_nvfp4(xp, xs, gx, perm, offsets, k, wp, ws, gw, gy)
    used = int(offsets[-1])
    back = O.dequantize(packed[:used], scales[:used], gy)
    yb = y[:used].reshape(used, -1, 16)
    err = np.abs(back.reshape(used, -1, 16) - yb)
    amax = yb.max(axis=2, keepdims=True)
    assert (err <= 0.25 * amax * 1.01 + 1e-30).all()


# ---- SwiGLU --------------------------------------------------------------

def _small_swiglu_case(seed, T=5, k=3, E=4, K=32, N=32):
    """As _small_case, with 2N weight rows (gate rows, then up rows) and
    power-of-two global scales, so every FC1 value is exact in float64
    whatever the order of its sum."""
    xp, xs, gx, perm, offsets, k, wp, ws, gw = _small_case(seed, T=T, k=k, E=E, K=K, N=2 * N)
    gw = (2.0 ** (np.arange(E) % 4 - 1)).astype(np.float32)
    return xp, xs, np.float32(2.0), perm, offsets, k, wp, ws, gw


def test_silu_closed_forms():
    """silu(g) = g sigmoid(g): sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4
    exactly; sigmoid(g) + sigmoid(-g) = 1 gives silu(g) - silu(-g) = g; the
    function's minimum, at g* = -1 - W(1/e), equals g* + 1; far from 0 it is
    g itself above and a tiny negative number below."""
    ln3 = np.log(3.0)
    assert O.silu(0.0) == 0.0
    assert O.silu(ln3) == pytest.approx(0.75 * ln3, rel=1e-15)
    assert O.silu(-ln3) == pytest.approx(-0.25 * ln3, rel=1e-15)
    g = np.concatenate([np.linspace(-60, 60, 241), [1e-30, 700.0, -700.0]])
    assert np.allclose(O.silu(g) - O.silu(-g), g, rtol=1e-15, atol=1e-300)
    assert O.silu(O.SILU_ARGMIN) == pytest.approx(O.SILU_ARGMIN + 1.0, abs=1e-15)
    grid = np.linspace(-5, 5, 200001)
    assert O.silu(grid).min() >= O.silu(O.SILU_ARGMIN)
    assert abs(grid[np.argmin(O.silu(grid))] - O.SILU_ARGMIN) <= 1e-4
    assert O.silu(40.0) == 40.0
    s = O.silu(-40.0)
    assert s < 0 and s == pytest.approx(-40.0 * np.exp(-40.0), rel=1e-15)
    assert O.silu(-800.0) == 0.0                          # underflows, never overflows
    assert O.swiglu(2.0, 3.0) == pytest.approx(2.0 * 3.0 / (1.0 + np.exp(-2.0)), rel=1e-15)


def test_swiglu_matches_a_written_out_loop():
    """Output column n of grouped row p is silu(gate) * up with gate from
    weight row n and up from weight row N + n of the row's expert, each a
    sum over k of table-decoded products; the FP32 result is then quantised
    (the pinned pre-expert quantiser)."""
    xp, xs, gx, perm, offsets, k, wp, ws, gw = _small_swiglu_case(13)
    K, N2 = xp.shape[1] * 2, wp.shape[1]
    N = N2 // 2
    E = len(offsets) - 1
    y = np.zeros((len(perm), N))
    for p in range(int(offsets[-1])):
        e = max(i for i in range(E) if offsets[i] <= p)
        t = perm[p] // k
        for n in range(N):
            gate = sum(_decode(xp[t], xs[t], gx, i) * _decode(wp[e, n], ws[e, n], gw[e], i) for i in range(K))
            up = sum(_decode(xp[t], xs[t], gx, i) * _decode(wp[e, N + n], ws[e, N + n], gw[e], i) for i in range(K))
            y[p, n] = gate / (1.0 + np.exp(-gate)) * up
    gy = O.global_scale(y)
    ref_p, ref_s = O.nvfp4_quantize(y.astype(np.float32), gy)
    used = int(offsets[-1])
    ref_p[used:] = 0
    ref_s[used:] = 0
    got_p, got_s = O.expert_fc1_swiglu_nvfp4(xp, xs, gx, perm, offsets, k, wp, ws, gw, gy)
    assert got_p.shape == (len(perm), N // 2) and got_s.shape == (len(perm), N // 16)
    assert np.array_equal(got_p, ref_p) and np.array_equal(got_s, ref_s)


def _one_hot_swiglu(cols, gw=1.0):
    """K = 16 input one-hot at k = 0 with value 1: output column n's gate is
    weight (n, 0) and its up weight (N + n, 0). cols: {n: (gate byte, gate
    scale byte, up byte, up scale byte)} (code in the low nibble)."""
    K, N = 16, 16
    xp = np.zeros((1, K // 2), dtype=np.uint8)
    xp[0, 0] = 0x02
    xs = np.array([[0x38]], dtype=np.uint8)
    wp = np.zeros((1, 2 * N, K // 2), dtype=np.uint8)
    ws = np.full((1, 2 * N, 1), 0x38, dtype=np.uint8)
    for n, (gc, gsb, uc, usb) in cols.items():
        wp[0, n, 0], ws[0, n, 0] = gc, gsb
        wp[0, N + n, 0], ws[0, N + n, 0] = uc, usb
    args = (xp, xs, 1.0, np.array([0], np.int32), np.array([0, 1], np.int32), 1, wp, ws,
            np.array([gw], np.float32))
    return args


def test_swiglu_one_hot_gate_and_up_order():
    """Gate 2, up 3: y = 6 sigmoid(2) = 5.2848 is the block maximum; 5.2848 *
    RN32(1/6) = 0.8808 rounds to E4M3 0.875 (0x36), so out = 1/0.875 and
    q = 6.0398 saturates to code 7. Gate 0.5, up -4: y = -2 sigmoid(0.5) =
    -1.2449, q = -1.4228, code 1.5 with the sign (0xB). Gate -2, up 3:
    y = -6 sigmoid(-2) = -0.7152, q = -0.8174, code 1.0 with the sign (0xA).
    Swapping gate and up would give 6 sigmoid(3) = 5.7155 as the maximum and
    scale 0.9375 (0x37) instead."""
    args = _one_hot_swiglu({0: (0x04, 0x38, 0x05, 0x38), 1: (0x01, 0x38, 0x0E, 0x38),
                            2: (0x0C, 0x38, 0x05, 0x38)})
    acc, _ = O.fc1_exact(*args)
    assert list(acc[0, :3]) == [2.0, 0.5, -2.0] and list(acc[0, 16:19]) == [3.0, -4.0, 3.0]
    packed, scales = O.expert_fc1_swiglu_nvfp4(*args, 1.0)
    assert scales[0, 0] == 0x36
    codes = [(packed[0, i // 2] >> (4 * (i % 2))) & 15 for i in range(16)]
    assert codes == [7, 0xB, 0xA] + [0] * 13
    assert not O.fc1_swiglu_boundary_blocks(*args, 1.0)[0, 0]


def test_swiglu_boundary_set():
    """Values far from every threshold are not flagged. A tiny negative value
    whose FP32 evaluation may underflow to zero, and so lose the sign bit,
    is: with gs_w = 0.1, gate -6 * 1.75 / 0.1 = -105 and up 2 / 0.1 = 20
    give y = -8.4e-43, a nonzero FP32 subnormal (code 0x8, negative zero),
    next to a column with gate and up 20 (y = 400)."""
    # far from thresholds: gate 2, up 2 -> 4 sigmoid(2) = 3.5232 (block max,
    # scale 0.5859 -> 0x33 = 0.5625, q = 6.26 -> 7); gate 1, up 1 -> 0.7311,
    # q = 1.30 (between 1.25 and 1.75)
    args = _one_hot_swiglu({0: (0x04, 0x38, 0x04, 0x38), 1: (0x02, 0x38, 0x02, 0x38)})
    assert not O.fc1_swiglu_boundary_blocks(*args, 1.0)[0, 0]
    # a gate of exactly 0 gives y = 0 exactly, which is not flagged either
    args = _one_hot_swiglu({0: (0x04, 0x38, 0x04, 0x38), 1: (0x00, 0x38, 0x05, 0x38)})
    assert not O.fc1_swiglu_boundary_blocks(*args, 1.0)[0, 0]
    args = _one_hot_swiglu({0: (0x0F, 0x3E, 0x04, 0x38), 1: (0x04, 0x38, 0x04, 0x38)}, gw=0.1)
    acc, _ = O.fc1_exact(*args)
    y = O.swiglu(acc[0, :2], acc[0, 16:18]).astype(np.float32)
    assert y[0] < 0 and y[0] > -1e-40 and y[1] == pytest.approx(400.0, rel=1e-6)
    packed, scales = O.expert_fc1_swiglu_nvfp4(*args, 1.0)
    assert packed[0, 0] & 15 == 0x8
    assert O.fc1_swiglu_boundary_blocks(*args, 1.0)[0, 0]
    # the same block without the tiny value is not flagged
    args = _one_hot_swiglu({1: (0x04, 0x38, 0x04, 0x38)}, gw=0.1)
    assert not O.fc1_swiglu_boundary_blocks(*args, 1.0)[0, 0]


def test_swiglu_boundary_set_flags_a_threshold_tie():
    """On FC1 values directly: column 0 gives y = 6 (gate 30, up 6 / silu(30)
    = 6 within an ulp), so with gs_y = 1 the block scale is 6 * RN32(1/6) =
    1.0 exactly and out = 1; column 1's y is then its own code input q. With
    y = 2.5 (the printed threshold between codes 4 and 5) the block is
    flagged, with y = 2.0 (between the thresholds 1.75 and 2.5) it is not,
    nor with the up value 1e-3 away from the tie."""
    def near_for(y1):
        acc = np.zeros((1, 32))
        acc[0, 0], acc[0, 16] = 30.0, 6.0 / O.silu(30.0)
        acc[0, 1], acc[0, 17] = 2.0, y1 / O.silu(2.0)
        return O.swiglu_boundary_from_values(acc, np.abs(acc), 64, 1.0)[0, 0]
    assert near_for(2.5)
    assert not near_for(2.0)
    assert not near_for(2.5 * (1 + 1e-3)) and not near_for(2.5 * (1 - 1e-3))


def test_swiglu_quantised_output_within_the_block_error_bound():
    """The dequantised output is within a quarter of the block maximum of
    silu(gate) * up (NVFP4's worst case)."""
    xp, xs, gx, perm, offsets, k, wp, ws, gw = _small_swiglu_case(21, T=8, k=4, E=6, K=64, N=48)
    acc, _ = O.fc1_exact(xp, xs, gx, perm, offsets, k, wp, ws, gw)
    N = acc.shape[1] // 2
    y = O.swiglu(acc[:, :N], acc[:, N:])
    gy = O.global_scale(y)
    packed, scales = O.expert_fc1_swiglu_nvfp4(xp, xs, gx, perm, offsets, k, wp, ws, gw, gy)
    used = int(offsets[-1])
    back = O.dequantize(packed[:used], scales[:used], gy)
    yb = y[:used].reshape(used, -1, 16)
    err = np.abs(back.reshape(used, -1, 16) - yb)
    amax = np.abs(yb).max(axis=2, keepdims=True)
    assert (err <= 0.25 * amax * 1.01 + 1e-30).all()
    assert not packed[used:].any() and not scales[used:].any()
