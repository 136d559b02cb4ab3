"""moe_norm_quant_nvfp4 against the oracle: codes and scales bit-exact
outside the stated set of BF16-midpoint blocks, within one step inside it;
exact everywhere on power-of-two rows; every workload shape."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as wl
from gpu_helpers import check_nvfp4, dev, e2m1_step_distance, host, note, require_gpu, scalar_dev, unpack_codes

pytestmark = pytest.mark.gpu

m = pytest.importorskip("moe_token_routing_amd")


def _run(x, nw, gc, eps, gs, what):
    require_gpu()
    note("norm_quant %s T=%d H=%d" % (what, x.shape[0], x.shape[1]))
    packed, scales = m.norm_quant_nvfp4(dev(x), dev(nw), gc, eps, scalar_dev(gs))
    torch.cuda.synchronize()
    return host(packed), host(scales)


def _check(x, nw, gc, eps, gs, got_packed, got_scales, rows, what):
    return check_nvfp4(x[rows], nw, gc, eps, gs, got_packed[rows], got_scales[rows], what)


@pytest.mark.parametrize("name,T", [("tiny", None), ("decode", None), ("prefill", 257),
                                    ("large_e", 100), ("wide_k", 5001)])
def test_norm_quant_workloads(name, T):
    w = wl.WORKLOADS[name]
    T = w.T if T is None else T
    x = wl.quant_input(w, T)
    nw = wl.quant_gain(w)
    y = O.rmsnorm_bf16(x, nw, w.quant_gain_center, w.eps)
    gs = O.global_scale(y)
    p, s = _run(x, nw, w.quant_gain_center, w.eps, gs, name)
    nset, nmis = _check(x, nw, w.quant_gain_center, w.eps, gs, p, s, np.arange(T), name)
    print("%s: stated-set blocks %d of %d, code mismatches inside %d" % (name, nset, s.size, nmis))


def test_norm_quant_prefill_full_size():
    """Every row of the 8192-token prefill batch."""
    w = wl.WORKLOADS["prefill"]
    x = wl.quant_input(w)
    nw = wl.quant_gain(w)
    gs = O.global_scale(O.rmsnorm_bf16(x, nw, w.quant_gain_center, w.eps))
    p, s = _run(x, nw, w.quant_gain_center, w.eps, gs, "prefill-full")
    nset, nmis = _check(x, nw, w.quant_gain_center, w.eps, gs, p, s, np.arange(w.T), "prefill-full")
    print("prefill-full: stated-set blocks %d of %d, code mismatches inside %d" % (nset, s.size, nmis))


def test_norm_quant_power_of_two_rows_exact():
    """Rows of +-2^m with eps = 0 normalise exactly to +-gain; gains sweep the
    E2M1 thresholds and every E4M3 scale regime (global scale varied)."""
    g = np.random.default_rng(50)
    H = 1024
    T = 48
    signs = g.choice([-1.0, 1.0], (T, H))
    x = wl.f32_to_bf16_bits((signs * 2.0 ** g.integers(-6, 6, (T, 1))).astype(np.float32))
    grid = np.array([0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0, 7.0])
    gains = np.tile(grid, H // 16) * 2.0 ** np.repeat(g.integers(-8, 8, H // 16), 16)
    nw = O.round_bf16(gains).astype(np.float32)
    assert not O.midpoint_boundary_blocks(x, nw, 0.0, 0.0).any()
    for gs in (1.0, 448.0 * 6 / 7.0 * 2 ** -8, 3.0e-3, 1e5, 0.7):
        p, s = _run(x, nw, 0.0, 0.0, gs, "pow2 gs=%g" % gs)
        rp, rs = O.norm_quant_nvfp4(x, nw, 0.0, 0.0, gs)
        np.testing.assert_array_equal(s, rs)
        np.testing.assert_array_equal(p, rp)


@pytest.mark.parametrize("H", [16, 48, 272, 1024, 2064, 4096, 16384])
def test_norm_quant_widths(H):
    g = np.random.default_rng(H + 1)
    T = 29
    x = wl.f32_to_bf16_bits((g.standard_normal((T, H)) * 3).astype(np.float32))
    x[3] = 0                                           # an all-zero row
    x[4, :16] = 0x8000                                 # negative zeros
    nw = g.uniform(-1, 1, H).astype(np.float32)
    gs = O.global_scale(O.rmsnorm_bf16(x, nw, 1.0, 1e-6))
    p, s = _run(x, nw, 1.0, 1e-6, gs, "H=%d" % H)
    _check(x, nw, 1.0, 1e-6, gs, p, s, np.arange(T), "H=%d" % H)
    assert (s[3] == 0).all() and (p[3] == 0).all()


@pytest.mark.parametrize("T,H", [(9001, 1024), (4000, 4096), (3000, 8192), (1500, 12288), (1000, 16384)])
def test_norm_quant_blocks_visit_several_tokens(T, H):
    """Token counts past what fits on the GPU at once (256 CUs at up to 8
    waves per SIMD: 2048 blocks of 4 waves) for every width whose tokens fill
    whole waves (H = 1024: four tokens per block) or the whole block (H a
    multiple of 4096): blocks then loop over several tokens and copy each
    next row into LDS ahead. Ragged counts leave blocks with one token fewer
    and, at H = 1024, a last block with idle waves. Every row checked."""
    g = np.random.default_rng(T + H)
    x = wl.f32_to_bf16_bits((g.standard_normal((T, H)) * 3).astype(np.float32))
    x[T - 1] = 0                                       # an all-zero last row
    x[T // 2, 16:32] = 0x8000                          # negative zeros
    nw = g.uniform(-1, 1, H).astype(np.float32)
    gs = O.global_scale(O.rmsnorm_bf16(x, nw, 1.0, 1e-6))
    p, s = _run(x, nw, 1.0, 1e-6, gs, "several tokens per block")
    _check(x, nw, 1.0, 1e-6, gs, p, s, np.arange(T), "T=%d H=%d" % (T, H))
    assert (s[T - 1] == 0).all() and (p[T - 1] == 0).all()
    if H == 8192:
        pooled = _gather_shards(x, 4)
        note("norm_quant rank block T=%d H=%d tp=4" % (T, H))
        pr, sr = m.norm_quant_nvfp4_rank_block(dev(pooled), T, dev(nw), 1.0, 1e-6, scalar_dev(gs))
        torch.cuda.synchronize()
        assert np.array_equal(host(pr), p) and np.array_equal(host(sr), s)


def test_norm_quant_zero_tokens():
    require_gpu()
    p, s = m.norm_quant_nvfp4(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda:0"),
                              torch.ones(64, dtype=torch.float32, device="cuda:0"), 1.0, 1e-6,
                              scalar_dev(1.0))
    assert p.shape == (0, 32) and s.shape == (0, 4)


def _gather_shards(x, tp):
    """The rank-block input a dim-0 all-gather of tp column shards leaves."""
    S = x.shape[1] // tp
    return np.ascontiguousarray(np.concatenate([x[:, r * S:(r + 1) * S] for r in range(tp)], axis=0))


@pytest.mark.parametrize("name,T,tp", [("prefill", 300, 2), ("prefill", 300, 8), ("prefill", 64, 512),
                                       ("wide_k", 1001, 4), ("wide_k", 1001, 64), ("tiny", None, 4)])
def test_norm_quant_rank_block(name, T, tp):
    """Rank-block input [tp*T, H/tp]: identical bytes to the contiguous call
    on the same logical rows, and the oracle's parity rule on them."""
    require_gpu()
    w = wl.WORKLOADS[name]
    T = w.T if T is None else T
    x = wl.quant_input(w, T)
    nw = wl.quant_gain(w)
    y = O.rmsnorm_bf16(x, nw, w.quant_gain_center, w.eps)
    gs = O.global_scale(y)
    pooled = _gather_shards(x, tp)
    note("norm_quant rank block %s T=%d H=%d tp=%d" % (name, T, w.H, tp))
    p, s = m.norm_quant_nvfp4_rank_block(dev(pooled), T, dev(nw), w.quant_gain_center, w.eps, scalar_dev(gs))
    torch.cuda.synchronize()
    p, s = host(p), host(s)
    pc, sc = _run(x, nw, w.quant_gain_center, w.eps, gs, name + " contiguous")
    assert np.array_equal(p, pc) and np.array_equal(s, sc)
    _check(x, nw, w.quant_gain_center, w.eps, gs, p, s, np.arange(T), name + " rank block")


def test_norm_quant_rank_block_full_prefill_sampled():
    """The prefill batch (T=8192, H=8192) as an 8-way rank block, sampled rows
    against the oracle."""
    require_gpu()
    w = wl.WORKLOADS["prefill"]
    x = wl.quant_input(w)
    nw = wl.quant_gain(w)
    gs = np.float32(345.4457702636719)
    pooled = _gather_shards(x, 8)
    note("norm_quant rank block prefill full tp=8")
    p, s = m.norm_quant_nvfp4_rank_block(dev(pooled), w.T, dev(nw), w.quant_gain_center, w.eps, scalar_dev(gs))
    torch.cuda.synchronize()
    rows = np.random.default_rng(7).choice(w.T, 64, replace=False)
    _check(x, nw, w.quant_gain_center, w.eps, gs, host(p), host(s), np.sort(rows), "prefill rank block")
