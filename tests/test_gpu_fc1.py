"""moe_expert_fc1_nvfp4 against the oracle: codes and scales bit-exact
outside the boundary set (blocks an FP32 accumulation may legitimately
change), within one step inside it; zero rows past the routed count; empty
and many-tile experts; the FC1 workload the act-fusion GEMM page times
(K 1024, N 2688, 512 experts, top-22) at full size, sampled."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as wl
from gpu_helpers import dev, e2m1_step_distance, host, note, require_gpu, scalar_dev, unpack_codes

pytestmark = pytest.mark.gpu

m = pytest.importorskip("moe_token_routing_amd")


def _routing(g, T, k, E, invalid=0.0, skew=None):
    ids = np.empty((T, k), dtype=np.int32)
    p = None
    if skew is not None:
        p = np.asarray(skew, dtype=np.float64)
        p = p / p.sum()
    for t in range(T):
        ids[t] = g.choice(E, size=k, replace=False, p=p)
    if invalid:
        ids[g.uniform(size=(T, k)) < invalid] = -1
    counts, offsets, perm, dest = O.dispatch(ids, E)
    return perm.astype(np.int32), offsets.astype(np.int32)


def _run(xp, xs, gx, perm, offsets, k, wp, ws, gw, gy, what):
    require_gpu()
    note("fc1 %s T=%d K=%d N=%d E=%d k=%d" % (what, xp.shape[0], xp.shape[1] * 2, wp.shape[1], wp.shape[0], k))
    yp, ys = m.expert_fc1_nvfp4(dev(xp), dev(xs), scalar_dev(gx), dev(perm), dev(offsets), k,
                                dev(wp), dev(ws), dev(gw), scalar_dev(gy))
    torch.cuda.synchronize()
    return host(yp), host(ys)


def _check(got_p, got_s, ref_p, ref_s, near, what):
    gc, rc = unpack_codes(got_p), unpack_codes(ref_p)
    nearel = np.repeat(near, 16, axis=1)
    assert np.array_equal(got_s[~near], ref_s[~near]), what + ": scale mismatch outside the boundary set"
    bad = (gc != rc) & ~nearel
    assert not bad.any(), "%s: %d code mismatches outside the boundary set" % (what, int(bad.sum()))
    if near.any():
        assert (np.abs(got_s[near].astype(int) - ref_s[near].astype(int)) <= 1).all()
        assert (e2m1_step_distance(gc[nearel], rc[nearel]) <= 1).all()
    return int(near.sum()), int(((gc != rc) & nearel).sum())


def _case(T, k, E, K, N, seed, invalid=0.0, skew=None):
    g = np.random.default_rng(seed)
    w = wl.WORKLOADS["wide_k"]
    xp, xs = wl.fc1_activations(w, T, K)
    wp, ws, gw = wl.fc1_weights(w, N, E, K)
    perm, offsets = _routing(g, T, k, E, invalid, skew)
    gx = np.float32(37.5)
    acc, _ = O.fc1_exact(xp, xs, gx, perm, offsets, k, wp, ws, gw)
    gy = O.global_scale(O.relu2(acc))
    return xp, xs, gx, perm, offsets, k, wp, ws, gw, gy


@pytest.mark.parametrize("T,k,E,K,N,invalid,skew", [
    (37, 3, 5, 128, 256, 0.1, None),            # ragged tiles, invalid slots
    (300, 2, 4, 64, 128, 0.0, [10, 0, 1, 3]),   # an empty expert, one expert over several tiles
    (64, 4, 16, 256, 384, 0.0, None),           # many small experts
    (40, 2, 3, 576, 384, 0.0, None),            # 9 K stages: a second scale chunk of one stage
    (33, 3, 5, 1088, 256, 0.05, None),          # 17 K stages: a third chunk, a partial scale row
    (9, 2, 2, 16384, 128, 0.0, None),           # the largest K: 256 stages, 32 scale chunks
    # from 1024 routed rows an expert the 256-row tiles (above: 128 x 128)
    (1100, 2, 2, 128, 384, 0.0, None),          # 256 x 192
    (1100, 2, 2, 128, 256, 0.02, None),         # 256 x 256
    (1100, 2, 2, 128, 128, 0.0, [3, 1]),        # 256 x 128, uneven experts
])
def test_fc1_small(T, k, E, K, N, invalid, skew):
    args = _case(T, k, E, K, N, seed=T + E, invalid=invalid, skew=skew)
    xp, xs, gx, perm, offsets, k, wp, ws, gw, gy = args
    got_p, got_s = _run(*args, "small")
    ref_p, ref_s = O.expert_fc1_nvfp4(*args)
    near = O.fc1_boundary_blocks(*args)
    nset, nmis = _check(got_p, got_s, ref_p, ref_s, near, "fc1")
    used = int(offsets[-1])
    assert not got_p[used:].any() and not got_s[used:].any()
    print("boundary blocks %d of %d, code mismatches inside %d" % (nset, near.size, nmis))


def test_fc1_deterministic():
    args = _case(100, 3, 6, 128, 256, seed=4)
    a = _run(*args, "determinism 1")
    b = _run(*args, "determinism 2")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_fc1_zero_tokens():
    require_gpu()
    E, K, N = 4, 64, 128
    yp, ys = m.expert_fc1_nvfp4(torch.zeros((0, K // 2), dtype=torch.uint8, device="cuda"),
                                torch.zeros((0, K // 16), dtype=torch.uint8, device="cuda"),
                                scalar_dev(1.0), torch.zeros(0, dtype=torch.int32, device="cuda"),
                                torch.zeros(E + 1, dtype=torch.int32, device="cuda"), 2,
                                torch.zeros((E, N, K // 2), dtype=torch.uint8, device="cuda"),
                                torch.zeros((E, N, K // 16), dtype=torch.uint8, device="cuda"),
                                torch.ones(E, dtype=torch.float32, device="cuda"), scalar_dev(1.0))
    assert yp.shape == (0, N // 2) and ys.shape == (0, N // 16)


def test_fc1_full_workload_sampled():
    """T = 32768 tokens, top-22 of 512 experts, K 1024, N 2688, at full size;
    rows of 6 experts checked against the oracle."""
    require_gpu()
    w = wl.WORKLOADS["wide_k"]
    T, k, E, K, N = w.T, w.k, w.E, w.H, wl.FC1_N["wide_k"]
    xp, xs = wl.fc1_activations(w, T, K)
    wp, ws, gw = wl.fc1_weights(w, N, E, K)
    ids = wl.synthetic_topk_ids(w, T)
    counts, offsets, perm, dest = O.dispatch(ids, E)
    perm, offsets = perm.astype(np.int32), offsets.astype(np.int32)
    gx = np.float32(37.5)
    g = np.random.default_rng(11)
    experts = g.choice(E, size=6, replace=False)
    rows = np.concatenate([np.arange(offsets[e], offsets[e + 1])[:24] for e in experts])
    # the sampled rows as a problem of their own: same tokens and experts
    sub_ids = np.full((len(rows), 1), -1, dtype=np.int32)
    sub_exp = np.array([np.searchsorted(offsets, r, side="right") - 1 for r in rows])
    sub_ids[:, 0] = sub_exp
    c2, off2, perm2, _ = O.dispatch(sub_ids, E)
    tok = perm[rows] // k
    sx_p, sx_s = xp[tok], xs[tok]
    sub_args = (sx_p, sx_s, gx, perm2.astype(np.int32), off2.astype(np.int32), 1, wp, ws, gw)
    acc, _ = O.fc1_exact(*sub_args)
    gy = O.global_scale(O.relu2(acc))
    ref_p, ref_s = O.expert_fc1_nvfp4(*sub_args, gy)
    near = O.fc1_boundary_blocks(*sub_args, gy)
    got_p, got_s = _run(xp, xs, gx, perm, offsets, k, wp, ws, gw, gy, "wide_k full")
    # sub-problem position q holds sampled row rows[perm2[q]]
    got_rows_p = got_p[rows[perm2]]
    got_rows_s = got_s[rows[perm2]]
    nset, nmis = _check(got_rows_p, got_rows_s, ref_p, ref_s, near, "fc1 wide_k")
    used = int(offsets[-1])
    assert used == T * k
    print("wide_k sampled rows %d: boundary blocks %d of %d, mismatches inside %d" % (len(rows), nset, near.size, nmis))


# ---- SwiGLU --------------------------------------------------------------

def _swiglu_values(acc):
    N = acc.shape[1] // 2
    return O.swiglu(acc[:, :N], acc[:, N:])


def _run_swiglu(xp, xs, gx, perm, offsets, k, wp, ws, gw, gy, what):
    require_gpu()
    note("fc1 swiglu %s T=%d K=%d N=%d E=%d k=%d" % (what, xp.shape[0], xp.shape[1] * 2, wp.shape[1] // 2,
                                                      wp.shape[0], k))
    yp, ys = m.expert_fc1_swiglu_nvfp4(dev(xp), dev(xs), scalar_dev(gx), dev(perm), dev(offsets), k,
                                       dev(wp), dev(ws), dev(gw), scalar_dev(gy))
    torch.cuda.synchronize()
    return host(yp), host(ys)


def _case_swiglu(T, k, E, K, N, seed, invalid=0.0, skew=None):
    g = np.random.default_rng(seed)
    w = wl.WORKLOADS["wide_k"]
    xp, xs = wl.fc1_activations(w, T, K)
    wp, ws, gw = wl.fc1_weights(w, 2 * N, E, K)
    perm, offsets = _routing(g, T, k, E, invalid, skew)
    gx = np.float32(37.5)
    acc, _ = O.fc1_exact(xp, xs, gx, perm, offsets, k, wp, ws, gw)
    gy = O.global_scale(_swiglu_values(acc))
    return xp, xs, gx, perm, offsets, k, wp, ws, gw, gy


@pytest.mark.parametrize("T,k,E,K,N,invalid,skew", [
    (37, 3, 5, 128, 64, 0.1, None),             # 128 weight rows per tile (64 columns), ragged, invalid slots
    (300, 2, 4, 64, 128, 0.0, [10, 0, 1, 3]),   # an empty expert, one over several row tiles
    (64, 4, 16, 256, 192, 0.0, None),           # many small experts
    (40, 2, 3, 576, 320, 0.0, None),            # five 128-row tiles over 640 weight rows, 9 K stages
    (33, 3, 5, 1088, 384, 0.05, None),          # 17 K stages, a partial scale row
    # from 1024 routed rows an expert the 256-row tiles (above: 128 x 128)
    (1100, 2, 2, 128, 192, 0.0, None),          # 256 x 192 (384 weight rows, 96 columns a tile)
    (1100, 2, 2, 128, 128, 0.02, None),         # 256 x 256 (128 columns)
    (1100, 2, 2, 128, 64, 0.0, [3, 1]),         # 256 x 128 (64 columns), uneven experts
])
def test_fc1_swiglu_small(T, k, E, K, N, invalid, skew):
    args = _case_swiglu(T, k, E, K, N, seed=T + E + 1, invalid=invalid, skew=skew)
    xp, xs, gx, perm, offsets, k, wp, ws, gw, gy = args
    got_p, got_s = _run_swiglu(*args, "small")
    ref_p, ref_s = O.expert_fc1_swiglu_nvfp4(*args)
    near = O.fc1_swiglu_boundary_blocks(*args)
    nset, nmis = _check(got_p, got_s, ref_p, ref_s, near, "fc1 swiglu")
    used = int(offsets[-1])
    assert got_p.shape == (T * k, N // 2)
    assert not got_p[used:].any() and not got_s[used:].any()
    # the output's signs: negative codes appear (silu and up both change sign)
    codes = unpack_codes(got_p[:used])
    assert (codes & 8).any() and (codes[codes > 0] & 7).any()
    print("boundary blocks %d of %d, code mismatches inside %d" % (nset, near.size, nmis))


def test_fc1_swiglu_tails():
    """Gate values far into silu's tails: the weights' global scales are
    small, so gate and up values reach the hundreds and beyond and silu(g)
    ranges from g itself (g > 0) through subnormal negative values (g in
    about -104..-87, whose FP32 evaluation may flush to zero: the boundary
    set flags those blocks) to an exact zero."""
    T, k, E, K, N = 48, 2, 3, 64, 64
    g = np.random.default_rng(5)
    w = wl.WORKLOADS["wide_k"]
    xp, xs = wl.fc1_activations(w, T, K)
    wp, ws, gw = wl.fc1_weights(w, 2 * N, E, K)
    gw = np.array([2.0 ** -6, 2.5, 0.5], np.float32)   # gates up to ~2e4, ~150 and ~800
    perm, offsets = _routing(g, T, k, E)
    gx = np.float32(4.0)
    args = (xp, xs, gx, perm, offsets, k, wp, ws, gw)
    acc, _ = O.fc1_exact(*args)
    assert acc[:, :N].min() < -100 and acc[:, :N].max() > 100
    gy = O.global_scale(_swiglu_values(acc))
    got_p, got_s = _run_swiglu(*args, gy, "tails")
    ref_p, ref_s = O.expert_fc1_swiglu_nvfp4(*args, gy)
    near = O.fc1_swiglu_boundary_blocks(*args, gy)
    nset, nmis = _check(got_p, got_s, ref_p, ref_s, near, "fc1 swiglu tails")
    print("boundary blocks %d of %d, code mismatches inside %d" % (nset, near.size, nmis))


def test_fc1_swiglu_and_relu2_share_the_grouping():
    """Same input, grouping and weight bytes: the SwiGLU call over 2N rows and
    the Relu2 call over the same 2N rows both leave the rows past the routed
    count zero and write every routed row."""
    args = _case_swiglu(50, 2, 4, 128, 128, seed=77, invalid=0.2)
    xp, xs, gx, perm, offsets, k, wp, ws, gw, gy = args
    sp, ss = _run_swiglu(*args, "grouping")
    rp, rs = _run(xp, xs, gx, perm, offsets, k, wp, ws, gw, gy, "grouping relu2")
    used = int(offsets[-1])
    assert used < len(perm)
    for p_, s_ in ((sp, ss), (rp, rs)):
        assert not p_[used:].any() and not s_[used:].any()
        assert (s_[:used] != 0).any(axis=1).all()


def test_fc1_swiglu_full_workload_sampled():
    """T = 32768 tokens, top-22 of 512 experts, K 1024, 1344 output columns
    over 2688 gate and up rows, at full size; rows of 6 experts checked
    against the oracle."""
    require_gpu()
    w = wl.WORKLOADS["wide_k"]
    T, k, E, K, N = w.T, w.k, w.E, w.H, wl.FC1_SWIGLU_N["wide_k"]
    xp, xs = wl.fc1_activations(w, T, K)
    wp, ws, gw = wl.fc1_weights(w, 2 * N, E, K)
    ids = wl.synthetic_topk_ids(w, T)
    counts, offsets, perm, dest = O.dispatch(ids, E)
    perm, offsets = perm.astype(np.int32), offsets.astype(np.int32)
    gx = np.float32(37.5)
    g = np.random.default_rng(12)
    experts = g.choice(E, size=6, replace=False)
    rows = np.concatenate([np.arange(offsets[e], offsets[e + 1])[:24] for e in experts])
    sub_ids = np.full((len(rows), 1), -1, dtype=np.int32)
    sub_ids[:, 0] = np.array([np.searchsorted(offsets, r, side="right") - 1 for r in rows])
    c2, off2, perm2, _ = O.dispatch(sub_ids, E)
    tok = perm[rows] // k
    sub_args = (xp[tok], xs[tok], gx, perm2.astype(np.int32), off2.astype(np.int32), 1, wp, ws, gw)
    acc, _ = O.fc1_exact(*sub_args)
    gy = O.global_scale(_swiglu_values(acc))
    ref_p, ref_s = O.expert_fc1_swiglu_nvfp4(*sub_args, gy)
    near = O.fc1_swiglu_boundary_blocks(*sub_args, gy)
    got_p, got_s = _run_swiglu(xp, xs, gx, perm, offsets, k, wp, ws, gw, gy, "wide_k full")
    nset, nmis = _check(got_p[rows[perm2]], got_s[rows[perm2]], ref_p, ref_s, near, "fc1 swiglu wide_k")
    assert int(offsets[-1]) == T * k
    print("wide_k sampled rows %d: boundary blocks %d of %d, mismatches inside %d" % (len(rows), nset, near.size, nmis))


def test_fc1_scale_bytes_full_range():
    """Input and weight scale bytes over the whole finite E4M3 range: zero
    blocks (0x00), every subnormal (0x01-0x07), normals up to 448 (0x7E),
    drawn uniformly; whole rows of zero scales and of 0x7E too."""
    g = np.random.default_rng(77)
    T, k, E, K, N = 64, 4, 8, 256, 256
    xp = g.integers(0, 256, size=(T, K // 2), dtype=np.uint8)
    xs = g.integers(0, 0x7F, size=(T, K // 16), dtype=np.uint8)
    xs[3] = 0x00                      # a token whose every block is zero
    xs[4] = 0x7E                      # every block at the largest scale
    xs[5] = g.integers(0, 8, size=K // 16)   # zero and subnormal scales only
    wp = g.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    ws = g.integers(0, 0x7F, size=(E, N, K // 16), dtype=np.uint8)
    ws[1, :7] = 0x00
    ws[2, 7:20] = 0x7E
    ws[3, 20:40] = g.integers(1, 8, size=(20, K // 16))
    gw = g.uniform(0.5, 8.0, size=E).astype(np.float32)
    perm, offsets = _routing(g, T, k, E, invalid=0.05)
    gx = np.float32(3.0)
    acc, _ = O.fc1_exact(xp, xs, gx, perm, offsets, k, wp, ws, gw)
    gy = O.global_scale(O.relu2(acc))
    args = (xp, xs, gx, perm, offsets, k, wp, ws, gw, gy)
    got_p, got_s = _run(*args, "scale bytes full range")
    ref_p, ref_s = O.expert_fc1_nvfp4(*args)
    near = O.fc1_boundary_blocks(*args)
    nset, nmis = _check(got_p, got_s, ref_p, ref_s, near, "fc1 scale range")
    used = int(offsets[-1])
    assert not got_p[used:].any() and not got_s[used:].any()
    assert (ref_s[:used] == 0x7E).any() and (ref_s[:used] == 0).any()
    print("boundary blocks %d of %d, code mismatches inside %d" % (nset, near.size, nmis))


@pytest.mark.parametrize("swiglu", [False, True])
def test_fc1_fed_by_the_pre_expert_quantiser(swiglu):
    """The chain the pages describe: moe_norm_quant_nvfp4's output, grouped
    by moe_dispatch of the routed ids, fed to the expert FC1 (TensorRT-LLM PR
    #21842, description; vLLM prepare_trtllm_nvfp4). The quantiser's scales
    here reach 448 (the static global scale puts the largest block there),
    E4M3 subnormals (a row of tiny values) and zero (an all-zero row). The
    quantiser is held to its rule against the oracle, and the FC1 to its rule
    on exactly the bytes the quantiser emitted."""
    require_gpu()
    g = np.random.default_rng(78)
    T, k, E, K, N = 96, 3, 6, 512, 256
    x = wl.f32_to_bf16_bits((g.standard_normal((T, K)) * 2).astype(np.float32))
    x[7] = 0                                                        # zero blocks
    x[8] = wl.f32_to_bf16_bits((g.standard_normal(K) * 1e-3).astype(np.float32))
    x[8, :16] = wl.f32_to_bf16_bits(np.full(16, 30.0, np.float32))  # one large block, the rest tiny
    x[9, 5] = wl.f32_to_bf16_bits(np.float32(400.0))                 # an outlier
    nw = g.uniform(-0.5, 0.5, K).astype(np.float32)
    gx = O.global_scale(O.rmsnorm_bf16(x, nw, 1.0, 1e-6))
    note("fc1 chain: norm_quant T=%d K=%d" % (T, K))
    xp_d, xs_d = m.norm_quant_nvfp4(dev(x), dev(nw), 1.0, 1e-6, scalar_dev(gx))
    ids = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[g.uniform(size=T) < 0.1] = -1                               # invalid tokens
    counts_d, offsets_d, perm_d, dest_d = m.dispatch(dev(ids), E)
    torch.cuda.synchronize()
    xp, xs = host(xp_d), host(xs_d)
    perm, offsets = host(perm_d), host(offsets_d)
    # the quantiser against its rule, the dispatch bit for bit
    from gpu_helpers import check_nvfp4
    check_nvfp4(x, nw, 1.0, 1e-6, gx, xp, xs, "chain quantiser")
    for got, want in zip((host(counts_d), offsets, perm, host(dest_d)), O.dispatch(ids, E)):
        np.testing.assert_array_equal(got, want)
    assert (xs == 0x7E).any() and (xs == 0).any() and ((xs > 0) & (xs < 8)).any()
    rows = 2 * N if swiglu else N
    wp = g.integers(0, 256, size=(E, rows, K // 2), dtype=np.uint8)
    ws = g.integers(0x30, 0x48, size=(E, rows, K // 16), dtype=np.uint8)
    gw = g.uniform(1.0, 4.0, size=E).astype(np.float32)
    fc1 = O.expert_fc1_swiglu_nvfp4 if swiglu else O.expert_fc1_nvfp4
    near_fn = O.fc1_swiglu_boundary_blocks if swiglu else O.fc1_boundary_blocks
    acc, _ = O.fc1_exact(xp, xs, gx, perm, offsets, k, wp, ws, gw)
    act = O.swiglu(acc[:, :N], acc[:, N:]) if swiglu else O.relu2(acc)
    gy = O.global_scale(act)
    note("fc1 chain: fc1 swiglu=%s" % swiglu)
    call = m.expert_fc1_swiglu_nvfp4 if swiglu else m.expert_fc1_nvfp4
    yp_d, ys_d = call(xp_d, xs_d, scalar_dev(gx), perm_d, offsets_d, k, dev(wp), dev(ws), dev(gw), scalar_dev(gy))
    torch.cuda.synchronize()
    args = (xp, xs, gx, perm, offsets, k, wp, ws, gw, gy)
    ref_p, ref_s = fc1(*args)
    near = near_fn(*args)
    nset, nmis = _check(host(yp_d), host(ys_d), ref_p, ref_s, near, "fc1 chain")
    print("chain swiglu=%s: boundary blocks %d of %d, mismatches inside %d" % (swiglu, nset, near.size, nmis))


# ---- inputs whose every partial sum is exact in FP32 ----------------------

_POW2_E4M3 = np.array([0x30, 0x38, 0x40], dtype=np.uint8)   # 0.5, 1, 2


def _case_dyadic(T, k, E, K, N, seed, invalid=0.0, skew=None, gx=4.0, gw_exp=(-2, 2)):
    """Uniform E2M1 codes with power-of-two block scales (E4M3 0.5, 1, 2) and
    power-of-two global scales: every dequantised element is a multiple of
    2^-2, every product of 2^-4, and while the sum of |products| stays below
    2^20 every partial sum, in any order and grouping, is a multiple of 2^-4
    below 2^20, so an FP32 accumulation rounds nowhere and alpha, a power of
    two, is exact too. The test asserts that premise on the drawn data."""
    g = np.random.default_rng(seed)
    xp = g.integers(0, 256, size=(T, K // 2), dtype=np.uint8)
    xs = _POW2_E4M3[g.integers(0, 3, size=(T, K // 16))]
    wp = g.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    ws = _POW2_E4M3[g.integers(0, 3, size=(E, N, K // 16))]
    gw = (2.0 ** g.integers(gw_exp[0], gw_exp[1] + 1, size=E)).astype(np.float32)
    gx = np.float32(gx)
    perm, offsets = _routing(g, T, k, E, invalid, skew)
    acc, mag = O.fc1_exact(xp, xs, gx, perm, offsets, k, wp, ws, gw)
    # undo alpha = 1 / (gs_x gs_w[e]) row by row: the kernel's raw sums
    used = int(offsets[-1])
    gw_row = np.zeros(len(perm))
    for e in range(E):
        gw_row[offsets[e]:offsets[e + 1]] = gw[e]
    raw_scale = (float(gx) * gw_row)[:, None]
    raw, raw_mag = acc * raw_scale, mag * raw_scale
    assert raw_mag[:used].max() * 16 < 2.0 ** 24, "premise: partial sums exact in FP32"
    assert np.array_equal(raw * 16, np.round(raw * 16)), "premise: multiples of 2^-4"
    return (xp, xs, gx, perm, offsets, k, wp, ws, gw), acc


@pytest.mark.parametrize("T,k,E,K,N,invalid,skew", [
    (9, 2, 2, 16384, 128, 0.0, None),           # the largest K: 256 stages, 32 scale chunks
    (300, 4, 8, 1024, 384, 0.05, [6, 0, 1, 1, 3, 1, 1, 2]),   # row tiles over experts, an empty one
    (37, 3, 5, 2048, 2688, 0.1, None),          # the FC1 workload's N: 14 column tiles
])
def test_fc1_dyadic_inputs_bit_exact(T, k, E, K, N, invalid, skew):
    """With exact accumulation the only rounding left is the square's (once,
    like the oracle's), so codes and scales must match on every block."""
    base, acc = _case_dyadic(T, k, E, K, N, seed=1000 + K, invalid=invalid, skew=skew)
    gy = O.global_scale(O.relu2(acc))
    args = base + (gy,)
    got_p, got_s = _run(*args, "dyadic")
    ref_p, ref_s = O.expert_fc1_nvfp4(*args)
    used = int(args[4][-1])
    assert np.array_equal(got_s, ref_s), "dyadic inputs: scale mismatch"
    assert np.array_equal(got_p, ref_p), "dyadic inputs: code mismatch"
    generic = O.fc1_boundary_blocks(*args)
    print("bit-exact on all %d blocks (the generic FP32 boundary set would excuse %d)"
          % (used * (N // 16), int(generic.sum())))


@pytest.mark.parametrize("T,k,E,K,N,invalid,gx", [
    (9, 2, 2, 16384, 64, 0.0, 128.0),
    (300, 4, 8, 1024, 192, 0.05, 32.0),
    (37, 3, 5, 2048, 1344, 0.1, 64.0),
])
def test_fc1_swiglu_dyadic_inputs(T, k, E, K, N, invalid, gx):
    """SwiGLU on the same exact-accumulation inputs: the gate and up values
    are exact, so the boundary set needs only the FP32 silu(g) u evaluation's
    error (no accumulation roundings). The global scales keep the gates
    within +-80, where silu stays a normal FP32 number, so no element is
    excused for an underflow."""
    base, acc = _case_dyadic(T, k, E, K, 2 * N, seed=2000 + K, invalid=invalid, gx=gx, gw_exp=(0, 2))
    assert np.abs(acc[:, :N]).max() < 80.0, "premise: gates within silu's normal range"
    gy = O.global_scale(_swiglu_values(acc))
    args = base + (gy,)
    got_p, got_s = _run_swiglu(*args, "dyadic")
    ref_p, ref_s = O.expert_fc1_swiglu_nvfp4(*args)
    near = O.fc1_swiglu_boundary_blocks(*args, adds=0)
    nset, nmis = _check(got_p, got_s, ref_p, ref_s, near, "fc1 swiglu dyadic")
    used = int(args[4][-1])
    assert not got_p[used:].any() and not got_s[used:].any()
    generic = O.fc1_swiglu_boundary_blocks(*args)
    print("boundary blocks %d of %d with exact sums (generic set %d), mismatches inside %d"
          % (nset, used * (N // 16), int(generic.sum()), nmis))
