"""The four calls chained on one stream at the full prefill shape (the
benchmark's workload and launch configuration), checked end to end against
the oracle on every token, and replayed inside a HIP graph -- on one stream
and with norm + quant forked onto a second stream -- with every replay
checked against the oracle and against an eager run.

TensorRT-LLM PR #21356, "Add the Muse Spark Open decoder fast paths": the
expert input is prepared on an auxiliary stream beside the routing ("Where
they plug in"), and each fused path is tested against the reference
composition and under CUDA graph replay with changed inputs (Test Coverage).
"""
import numpy as np
import pytest
import torch

import oracle as O
import route_checks as RC
import workloads as wl
from gpu_helpers import (DEV, check_combine, check_nvfp4, dev, host, note, require_gpu,
                         scalar_dev)

pytestmark = pytest.mark.gpu

m = pytest.importorskip("moe_token_routing_amd")


def _inputs(name, T=None):
    w = wl.WORKLOADS[name]
    T = w.T if T is None else T
    d = dict(w=w, T=T, hidden=wl.hidden(w, T), W=wl.router_weight(w), bias=wl.bias(w),
             mask=wl.token_mask(w, T), x=wl.quant_input(w, T), qw=wl.quant_gain(w),
             cg=wl.combine_gain(w), eo=wl.expert_out(w, T * w.k))
    return d


def _pipeline(d, gs):
    w = d["w"]
    lg, ids, tw = m.route(dev(d["hidden"]), dev(d["W"]), dev(d["bias"]), dev(d["mask"]), w.k)
    counts, offsets, perm, dest = m.dispatch(ids, w.E)
    packed, scales = m.norm_quant_nvfp4(dev(d["x"]), dev(d["qw"]), w.quant_gain_center, w.eps, scalar_dev(gs))
    out = m.combine(dev(d["eo"]), dest.view(d["T"], w.k), tw, dev(d["cg"]), 0.0, w.eps)
    torch.cuda.synchronize()
    return dict(lg=host(lg), ids=host(ids), tw=host(tw), counts=host(counts), offsets=host(offsets),
                perm=host(perm), dest=host(dest), packed=host(packed), scales=host(scales), out=host(out))


def _check_step(r, hidden, W, bias, mask, k, E, x, qw, qgc, eps, gs, eo, cg, route_rows, other_rows, what):
    """One step's outputs against the oracle: R1 on every token, R2 on
    route_rows, dispatch bit-exact, the NVFP4 and combine rules on
    other_rows (None: every row)."""
    T = mask.shape[0]
    ids_o, w_o = O.route_from_logits(r["lg"], bias, mask, k)
    np.testing.assert_array_equal(r["ids"], ids_o, err_msg=what + ": R1 ids")
    assert (np.abs(r["tw"].astype(np.float64) - w_o) <= 1e-5 * np.abs(w_o)).all(), what + ": R1 weights"
    lg_ref, mag = O.router_logits(hidden[route_rows], W)
    RC.assert_r2(r["lg"][route_rows], lg_ref, mag, mask[route_rows] != 0, what)
    for k_, rv in zip(("counts", "offsets", "perm", "dest"), O.dispatch(r["ids"], E)):
        np.testing.assert_array_equal(r[k_], rv, err_msg=what + ": dispatch " + k_)
    assert r["offsets"][-1] == int((mask != 0).sum()) * k
    rows = np.arange(T) if other_rows is None else other_rows
    check_nvfp4(x[rows], qw, qgc, eps, gs, r["packed"][rows], r["scales"][rows], what + ": nvfp4")
    slots = r["dest"].reshape(T, k)
    check_combine(eo, slots[rows], r["tw"][rows], cg, 0.0, eps, r["out"][rows], what + ": combine")


@pytest.mark.parametrize("name,T", [("prefill", None), ("wide_k", 4096)])
def test_pipeline_end_to_end(name, T):
    """Every token: R1, R2, dispatch, NVFP4 and combine against the oracle."""
    require_gpu()
    d = _inputs(name, T)
    w, T = d["w"], d["T"]
    gs = O.global_scale(O.rmsnorm_bf16(d["x"], d["qw"], w.quant_gain_center, w.eps))
    note("pipeline %s T=%d" % (name, T))
    r = _pipeline(d, gs)
    _check_step(r, d["hidden"], d["W"], d["bias"], d["mask"], w.k, w.E, d["x"], d["qw"], w.quant_gain_center,
                w.eps, gs, d["eo"], d["cg"], np.arange(T), None, "pipeline %s" % name)


@pytest.mark.parametrize("name", ["decode", "prefill"])
@pytest.mark.parametrize("two_stream", [False, True])
def test_pipeline_graph_replay(name, two_stream):
    """Capture the four calls in a HIP graph -- on one stream, or with norm +
    quant forked onto a second stream beside route -> dispatch -> combine --
    and replay it with new inputs copied into the captured buffers; every
    replay must equal a serial eager run bit for bit and meet the parity
    rules against the oracle (R1, dispatch on every token; R2, NVFP4 and
    combine on every token at 128 tokens, on 258 sampled tokens at 8192).
    At 128 tokens and at
    the 8192-token prefill batch, whose calls take their large-batch forms
    (weight planes split by a kernel of their own, tile histograms summed in
    the place step, norm + quant copying rows ahead, one block per token in
    the combine)."""
    require_gpu()
    w = wl.WORKLOADS[name]
    T = w.T
    d = _inputs(name)
    h_d, W_d, b_d, m_d = dev(d["hidden"]), dev(d["W"]), dev(d["bias"]), dev(d["mask"])
    x_d, qw_d, cg_d, eo_d = dev(d["x"]), dev(d["qw"]), dev(d["cg"]), dev(d["eo"])
    gs_d = scalar_dev(0.5)
    lg = torch.empty((T, w.E), dtype=torch.float32, device=DEV)
    ids = torch.empty((T, w.k), dtype=torch.int32, device=DEV)
    tw = torch.empty((T, w.k), dtype=torch.float32, device=DEV)
    ws_r = torch.empty(m.route_workspace_bytes(T, w.H, w.E, w.k, m.MOE_DTYPE_BF16), dtype=torch.uint8, device=DEV)
    ws_d = torch.empty(max(1, m.dispatch_workspace_bytes(T, w.k, w.E)), dtype=torch.uint8, device=DEV)
    counts = torch.empty(w.E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(w.E + 1, dtype=torch.int32, device=DEV)
    perm = torch.empty(T * w.k, dtype=torch.int32, device=DEV)
    dest = torch.empty(T * w.k, dtype=torch.int32, device=DEV)
    packed = torch.empty((T, w.H // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((T, w.H // 16), dtype=torch.uint8, device=DEV)
    out = torch.empty((T, w.H), dtype=torch.bfloat16, device=DEV)
    aux = torch.cuda.Stream()

    def norm_quant():
        m.norm_quant_nvfp4(x_d, qw_d, 1.0, w.eps, gs_d, packed=packed, scales=scales)

    def step():
        main = torch.cuda.current_stream()
        if two_stream:
            aux.wait_stream(main)
            with torch.cuda.stream(aux):
                norm_quant()
        m.route(h_d, W_d, b_d, m_d, w.k, logits=lg, topk_ids=ids, topk_w=tw, workspace=ws_r)
        m.dispatch(ids, w.E, counts=counts, offsets=offsets, perm=perm, dest=dest, workspace=ws_d)
        if not two_stream:
            norm_quant()
        m.combine(eo_d, dest.view(T, w.k), tw, cg_d, 0.0, w.eps, out=out)
        if two_stream:
            main.wait_stream(aux)

    def snapshot():
        return [host(t).copy() for t in (lg, ids, tw, counts, offsets, perm, dest, packed, scales, out)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    g = np.random.default_rng(12)
    for rep in range(3):
        note("graph replay %s %d (two_stream=%s)" % (name, rep, two_stream))
        # new inputs in place
        if name == "decode":
            h_d.copy_(dev(wl.f32_to_bf16_bits(g.standard_normal((T, w.H)).astype(np.float32))))
            x_d.copy_(dev(wl.f32_to_bf16_bits(g.standard_normal((T, w.H)).astype(np.float32))))
            mk = (g.uniform(size=T) > 0.2).astype(np.uint8)
            m_d.copy_(dev(mk))
        else:
            gt = torch.Generator(device=DEV).manual_seed(12 + rep)
            h_d.copy_(torch.randn((T, w.H), generator=gt, device=DEV).to(torch.bfloat16))
            x_d.copy_(torch.randn((T, w.H), generator=gt, device=DEV).to(torch.bfloat16))
            m_d.copy_((torch.rand(T, generator=gt, device=DEV) > 0.2).to(torch.uint8))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        replayed = snapshot()
        two = two_stream
        two_stream = False   # the eager reference runs serially on one stream
        step()
        two_stream = two
        torch.cuda.synchronize()
        eager = snapshot()
        for a, b in zip(replayed, eager):
            np.testing.assert_array_equal(a, b)
        # and the replay against the oracle on the inputs it was given
        r = dict(zip(("lg", "ids", "tw", "counts", "offsets", "perm", "dest", "packed", "scales", "out"), replayed))
        hidden_h, x_h, mask_h = host(h_d), host(x_d), host(m_d)
        if name == "decode":
            route_rows, other_rows = np.arange(T), None
        else:
            route_rows = other_rows = np.unique(np.concatenate([g.choice(T, 256, replace=False), [0, T - 1]]))
        _check_step(r, hidden_h, d["W"], d["bias"], mask_h, w.k, w.E, x_h, d["qw"], 1.0, w.eps, np.float32(0.5),
                    d["eo"], d["cg"], route_rows, other_rows,
                    "graph replay %s %d two_stream=%s" % (name, rep, two_stream))
