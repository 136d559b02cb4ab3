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
