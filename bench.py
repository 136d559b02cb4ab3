"""Benchmark of the MoE routing-and-combine hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill]
                    [--schedule fused|serial|prepare|overlap|overlap-route] [--graph]

One step is one pass of the whole path over one batch of synthetic input:
moe_route -> moe_dispatch -> moe_combine, and moe_norm_quant_nvfp4 (or
moe_route_dispatch in place of the first two, or moe_route_dispatch_quant in
place of the first three), with
inputs resident in HBM and every output and workspace allocated before the
timed region. The default workload is the 8192-token prefill batch (H=8192,
E=256, k=8, 5% invalid tokens). Prints one JSON line.

Schedules (the headline is the default `auto`: the prepare-fused schedule
launched eagerly):
  prepare-fused  moe_route_dispatch_quant (route, dispatch and the expert
                 input's norm + quant in one call; the dispatch's last step
                 and the norm + quant share one launch), then the combine
  fused          moe_route_dispatch (route and dispatch in one call, the
                 selection counting the dispatch's tile histograms), then
                 norm + quant and the combine, in order on one stream
  serial         the four calls in order on one stream
  prepare        norm + quant forked onto a second stream beside the dispatch
                 and joined before the combine (so it shares the GPU with
                 neither the projection nor the combine); the fork and join
                 cost more than the dispatch time they hide
  overlap        route on the main stream, then norm + quant forked onto a
                 second stream beside dispatch -> combine (it depends on none
                 of them); the step joins back into the main stream, so it
                 ends when both are done. Both sides are HBM-bound, so they
                 share the bandwidth rather than hide each other: about 5 us
                 slower per step than serial at the prefill shape
  overlap-route  norm + quant forked beside the route instead; the projection
                 is power-bound, so the two mostly slow each other down
  graph          the overlap step (and, reported beside it, the serial step)
                 captured once in a HIP graph and replayed; every kernel still
                 runs every step. At the prefill shape the replay is slower
                 than the eager overlap; at decode sizes, where launches
                 dominate, the serial graph is the fastest schedule

Before the W warm-up steps the headline step repeats, untimed, for 100 ms
(`clock_ramp` in the line): the GPU idles through the host-side setup and
needs ~15 ms of continuous work to reach its working clock.

Alongside the throughput the line carries:
  stages        per-call mean duration (HIP events on the launch stream, from
                a serial eager pass; route_dispatch from a fused pass) and
                algorithmic bytes / achieved GB/s
  schedules     ms per step of every schedule, and of the serial and the
                headline one with the 256 MB last-level cache flushed before
                each step (cold: by a 512 MiB write, and by a 512 MiB read,
                which leaves no dirty lines to write back); the p10 / median
                / p90 of single serial steps (HIP events)
  roofline      the dominant kernel (the combine) against MI355X's 8 TB/s:
                algorithmic bytes per launch / mean launch duration; `traffic`
                is the HBM bytes per launch from the committed rocprofv3
                counter summary, when that was taken on the current kernel
                source (null otherwise)
  expert_fc1    the expert FC1 (moe_expert_fc1_nvfp4) at the FC1 workload of
                the act-fusion GEMM page, against the FP16 MFMA peak (32768
                tokens; 8192 and 65536 tokens, the page's other two, beside)
  expert_fc1_swiglu  the SwiGLU form (moe_expert_fc1_swiglu_nvfp4) over the
                same 2688 weight rows as gate and up halves
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload,
                on the host cores this job may use, and on one core
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
RAMP_S = 0.1                    # untimed headline steps before the warm-up (GPU clock ramp)
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense FP16 / BF16 matrix peak
METRIC = "routed tokens/sec and % of HBM peak, H=8192 E=256 k=8, 8192 tokens"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "combine_prefill_traffic.json")
COMBINE_SRC = os.path.join(ROOT, "moe_token_routing_amd", "csrc", "combine.hip")


def algorithmic_bytes(w, hidden_bytes: int, valid_slots: int):
    """Bytes each call must move (inputs read once, outputs written once)."""
    T, H, E, k = w.T, w.H, w.E, w.k
    return {
        "route": T * H * hidden_bytes + E * H * 4 + E * 4 + T + T * k * 8,
        "dispatch": T * k * 4 * 3 + E * 4 + (E + 1) * 4,
        "norm_quant": T * H * 2 + H * 4 + T * H // 2 + T * H // 16,
        "combine": T * k * 8 + valid_slots * H * 2 + H * 4 + T * H * 2,
    }


def source_digest(path: str) -> str:
    h = hashlib.sha256()
    for p in sorted([path, os.path.join(os.path.dirname(path), "rows.hpp"),
                     os.path.join(os.path.dirname(path), "common.hpp")]):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per combine launch from the committed counter summary, if it
    was taken on this workload and on the current combine source."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("workload") != workload or d.get("source_digest") != source_digest(COMBINE_SRC):
        return None
    return d.get("bytes_per_launch")


def host_cores() -> int:
    """Cores this process may use: its CPU affinity, capped by OMP_NUM_THREADS
    when that is set (the share of the host a one-GPU job is given)."""
    n = len(os.sched_getaffinity(0))
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        cap = 0
    return min(n, cap) if cap > 0 else n


_CPU = {}   # the CPU baseline's inputs, set before its worker processes fork


def _cpu_route(rows):
    import oracle as O
    c = _CPU
    _, _, ids, tw = O.route(c["hidden"][rows], c["W"], c["bias"], c["mask"][rows], c["k"])
    return ids, tw


def _cpu_norm_quant(rows):
    import oracle as O
    c = _CPU
    return O.norm_quant_nvfp4(c["x"][rows], c["qw"], c["qgc"], c["eps"], np.float32(1.0))


def _cpu_combine(rows):
    import oracle as O
    c = _CPU
    return O.combine(c["eo"], c["dest"][rows], c["tw"][rows], c["cg"], 0.0, c["eps"])[0]   # the output rows


def cpu_baseline(w, sample_tokens: int, workers: int):
    """The oracle, as it stands, over the first `sample_tokens` tokens of the
    workload treated as one batch: route, dispatch, norm + quant, combine.
    With workers > 1 the per-token steps (route, norm + quant, combine) run on
    token chunks in that many forked processes and the dispatch, which sees
    every token, runs in the parent; BLAS is held to one thread per process.
    Call it before the GPU is initialised (it forks)."""
    import multiprocessing as mp

    import oracle as O
    import workloads as wl
    from threadpoolctl import threadpool_limits

    S = min(sample_tokens, w.T)
    _CPU.clear()
    _CPU.update(hidden=wl.hidden(w, S), W=wl.router_weight(w), bias=wl.bias(w), mask=wl.token_mask(w, S),
                k=w.k, x=wl.quant_input(w, S), qw=wl.quant_gain(w), qgc=w.quant_gain_center, eps=w.eps,
                cg=wl.combine_gain(w), eo=wl.expert_out(w, S * w.k))
    chunk = -(-S // max(1, workers))
    parts = [slice(a, min(S, a + chunk)) for a in range(0, S, chunk)]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        if workers > 1:
            pool = mp.get_context("fork").Pool(workers)
            try:
                r = pool.map(_cpu_route, parts)
                ids = np.concatenate([a for a, _ in r])
                _CPU["tw"] = np.concatenate([b for _, b in r])
                nq = pool.map_async(_cpu_norm_quant, parts)
                _, _, _, dest = O.dispatch(ids, w.E)
                nq.get()
                pool.close()
                pool.join()
                # the combine needs dest: fork a new pool that sees it
                _CPU["dest"] = dest.reshape(S, w.k)
                pool = mp.get_context("fork").Pool(workers)
                pool.map(_cpu_combine, parts)
            finally:
                pool.close()
                pool.join()
        else:
            ids, _CPU["tw"] = _cpu_route(slice(0, S))
            _, _, _, dest = O.dispatch(ids, w.E)
            _CPU["dest"] = dest.reshape(S, w.k)
            _cpu_norm_quant(slice(0, S))
            _cpu_combine(slice(0, S))
        dt = time.perf_counter() - t0
    _CPU.clear()
    how = ("route, norm + quant and combine on token chunks in %d processes, dispatch serial" % workers
           if workers > 1 else "one process, one thread")
    return {"value": round(S / dt, 1), "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": "first %d tokens of the %s workload as one batch, all four steps, %.1f s; %s"
                      % (S, w.name, dt, how)}


def time_expert_fc1(m, wl, torch, dev, stream, reps: int = 10, swiglu: bool = False, tokens=None):
    """The expert FC1 on the dispatched NVFP4 input at the FC1 workload the
    act-fusion GEMM page times (K 1024, N 2688, 512 experts, top-22, 32768
    tokens, or `tokens`): synthetic NVFP4 bytes, the path's own dispatch of
    synthetic top-22 ids, HIP events around each call. swiglu: the same 2688
    weight rows as gate and up halves (1344 output columns)."""
    w = wl.WORKLOADS["wide_k"]
    T, k, E, K = w.T if tokens is None else tokens, w.k, w.E, w.H
    N = wl.FC1_SWIGLU_N["wide_k"] if swiglu else wl.FC1_N["wide_k"]
    rows = 2 * N if swiglu else N
    xp, xs = wl.fc1_activations(w, T, K)
    wp, ws, gw = wl.fc1_weights(w, rows, E, K)
    ids = torch.from_numpy(wl.synthetic_topk_ids(w, T)).to(dev)
    X, XS = torch.from_numpy(xp).to(dev), torch.from_numpy(xs).to(dev)
    Wp, Ws, GW = torch.from_numpy(wp).to(dev), torch.from_numpy(ws).to(dev), torch.from_numpy(gw).to(dev)
    del xp, xs, wp, ws
    counts, offsets, perm, dest = m.dispatch(ids, E)
    gx = torch.tensor([37.5], dtype=torch.float32, device=dev)
    gy = torch.tensor([1.0e4], dtype=torch.float32, device=dev)
    yp = torch.empty((T * k, N // 2), dtype=torch.uint8, device=dev)
    ys = torch.empty((T * k, N // 16), dtype=torch.uint8, device=dev)
    wsp = torch.empty(m.expert_fc1_workspace_bytes(T, k, E), dtype=torch.uint8, device=dev)
    fn = m.expert_fc1_swiglu_nvfp4 if swiglu else m.expert_fc1_nvfp4

    def call():
        fn(X, XS, gx, perm, offsets, k, Wp, Ws, GW, gy, y_packed=yp, y_scales=ys, workspace=wsp)

    for _ in range(2):
        call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    flop = 2.0 * T * k * rows * K
    tf = flop / (ms * 1e-3) / 1e12
    what = ("SwiGLU, 1344 output columns over 2688 gate and up rows" if swiglu else "Relu2, N 2688")
    return {"workload": "K 1024, %s, 512 experts, top-22, %d tokens (%d routed rows)" % (what, T, T * k),
            "ms": round(ms, 3), "TFLOPs": round(tf, 1), "unit_peak_TFLOPs": MFMA_F16_PEAK_TFLOPS,
            "frac_of_fp16_mfma_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
            "bytes_in": int(T * K * 9 // 16 + E * rows * K * 9 // 16), "bytes_out": int(T * k * N * 9 // 16)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--cpu-sample", type=int, default=8192, help="tokens for the CPU oracle baseline (0: skip)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a 1 GiB device copy (a plain elementwise kernel) to calibrate HBM counters")
    ap.add_argument("--no-copy-ref", dest="copy_ref", action="store_false",
                    help="skip the 1 GiB device-copy reference bandwidth")
    ap.add_argument("--schedule", choices=["auto", "fused", "prepare-fused", "prepare", "overlap", "overlap-route",
                                           "serial"],
                    default="auto",
                    help="headline schedule: route, dispatch and norm+quant in one call then the combine "
                         "(prepare-fused), route and dispatch in one call then norm+quant and combine "
                         "(fused), the four calls on one stream (serial), norm+quant on a second stream "
                         "beside the dispatch (prepare), beside dispatch + combine (overlap) or beside the "
                         "route (overlap-route); auto = prepare-fused")
    ap.add_argument("--graph", action="store_true",
                    help="replay the headline schedule from a HIP graph instead of launching it eagerly")
    ap.add_argument("--no-fc1", dest="fc1", action="store_false",
                    help="skip timing the expert FC1 (K 1024, N 2688, 512 experts, top-22)")
    ap.add_argument("--stage", choices=["route", "dispatch", "route_dispatch", "route_dispatch_quant", "norm_quant",
                                        "combine"],
                    help="time one call of the path alone, repeated (after one fused step), then exit; "
                         "with --copy-calib also run a 1 GiB copy (for counter runs)")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="serial steps timed after flushing the last-level cache (0: skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import workloads as wl

    # the CPU oracle first: its worker processes fork, which must happen
    # before anything initialises the GPU
    cpu = None
    if args.cpu_sample > 0:
        cores = host_cores()
        cpu = cpu_baseline(wl.WORKLOADS[args.workload], args.cpu_sample, cores)
        # one core takes ~5x longer per token: a quarter of the sample
        cpu["one_core"] = (cpu_baseline(wl.WORKLOADS[args.workload], max(1, args.cpu_sample // 4), 1)
                           if cores > 1 else None)

    import torch
    import moe_token_routing_amd as m

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    m.lib()   # fails loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    w = wl.WORKLOADS[args.workload]
    T, H, E, k = w.T, w.H, w.E, w.k

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    with open(os.path.join(ROOT, "tests", "golden", "global_scales.json")) as f:
        gs_value = json.load(f)[w.name]["global_scale"]

    mask_np = wl.token_mask(w)
    hidden = to_dev(wl.hidden(w))
    W = to_dev(wl.router_weight(w))
    bias = to_dev(wl.bias(w))
    mask = to_dev(mask_np)
    x = to_dev(wl.quant_input(w))
    qw = to_dev(wl.quant_gain(w))
    cg = to_dev(wl.combine_gain(w))
    eo = to_dev(wl.expert_out(w))
    gs = torch.tensor([gs_value], dtype=torch.float32, device=dev)
    hdt = m.MOE_DTYPE_F32 if hidden.dtype == torch.float32 else m.MOE_DTYPE_BF16

    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, k), dtype=torch.float32, device=dev)
    ws_r = torch.empty(max(1, m.route_workspace_bytes(T, H, E, k, hdt)), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(max(1, m.dispatch_workspace_bytes(T, k, E)), dtype=torch.uint8, device=dev)
    ws_rd = torch.empty(max(1, m.route_dispatch_workspace_bytes(T, H, E, k, hdt)), dtype=torch.uint8, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    dest = torch.empty(T * k, dtype=torch.int32, device=dev)
    packed = torch.empty((T, H // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((T, H // 16), dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    slots = dest.view(T, k)
    stream = torch.cuda.current_stream(dev)

    def route_():
        m.route(hidden, W, bias, mask, k, logits=logits, topk_ids=ids, topk_w=tw, workspace=ws_r)

    def dispatch_():
        m.dispatch(ids, E, counts=counts, offsets=offsets, perm=perm, dest=dest, workspace=ws_d)

    def route_dispatch_():
        m.route_dispatch(hidden, W, bias, mask, k, logits=logits, topk_ids=ids, topk_w=tw, counts=counts,
                         offsets=offsets, perm=perm, dest=dest, workspace=ws_rd)

    def norm_quant_():
        m.norm_quant_nvfp4(x, qw, w.quant_gain_center, w.eps, gs, packed=packed, scales=scales)

    def route_dispatch_quant_():
        m.route_dispatch_quant(hidden, W, bias, mask, k, x, qw, w.quant_gain_center, w.eps, gs, logits=logits,
                               topk_ids=ids, topk_w=tw, counts=counts, offsets=offsets, perm=perm, dest=dest,
                               packed=packed, scales=scales, workspace=ws_rd)

    def combine_():
        m.combine(eo, slots, tw, cg, 0.0, w.eps, out=out)

    def step_serial(ev=None):
        main = torch.cuda.current_stream(dev)
        for j, call in enumerate((route_, dispatch_, norm_quant_, combine_)):
            if ev is not None:
                ev[j].record(main)
            call()
        if ev is not None:
            ev[4].record(main)

    def step_fused(ev=None):
        main = torch.cuda.current_stream(dev)
        for j, call in enumerate((route_dispatch_, norm_quant_, combine_)):
            if ev is not None:
                ev[j].record(main)
            call()
        if ev is not None:
            ev[3].record(main)

    def step_prepare_fused(ev=None):
        main = torch.cuda.current_stream(dev)
        for j, call in enumerate((route_dispatch_quant_, combine_)):
            if ev is not None:
                ev[j].record(main)
            call()
        if ev is not None:
            ev[2].record(main)

    aux = torch.cuda.Stream(device=dev)   # default priority

    def step_overlap_route():
        main = torch.cuda.current_stream(dev)
        aux.wait_stream(main)              # fork
        with torch.cuda.stream(aux):
            norm_quant_()
        route_()
        dispatch_()
        combine_()
        main.wait_stream(aux)              # join: the step ends when both are done

    def step_prepare():
        # norm + quant on the second stream beside the dispatch (latency-bound,
        # a few blocks), joined before the combine, so it never shares the
        # GPU with the projection or the combine's HBM stream
        main = torch.cuda.current_stream(dev)
        route_()
        aux.wait_stream(main)              # fork
        with torch.cuda.stream(aux):
            norm_quant_()
        dispatch_()
        main.wait_stream(aux)              # join before the combine
        combine_()

    def step_overlap():
        # the projection is power-bound, so norm + quant goes beside the
        # latency-bound dispatch and the combine rather than beside it
        main = torch.cuda.current_stream(dev)
        route_()
        aux.wait_stream(main)              # fork
        with torch.cuda.stream(aux):
            norm_quant_()
        dispatch_()
        combine_()
        main.wait_stream(aux)              # join

    def timed(fn, steps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1000.0 / steps

    if args.stage:
        # one call of the path, repeated (for counter runs): a fused step
        # first, so the dispatch and the combine see this batch's routing
        step_fused()
        call = {"route": route_, "dispatch": dispatch_, "route_dispatch": route_dispatch_,
                "route_dispatch_quant": route_dispatch_quant_, "norm_quant": norm_quant_,
                "combine": combine_}[args.stage]
        for _ in range(args.warmup):
            call()
        st = timed(call, args.steps)
        if args.copy_calib:
            ca = torch.zeros(1 << 29, dtype=torch.int16, device=dev)
            cb = torch.empty_like(ca)
            torch.neg(ca, out=cb)
            torch.cuda.synchronize()
            del ca, cb
        print(json.dumps({"stage": args.stage, "workload": w.name, "ms": round(st, 4), "steps": args.steps,
                          "copy_calib_GiB": 1 if args.copy_calib else 0}))
        return
    if args.schedule == "auto":
        args.schedule = "prepare-fused"
    head_step = {"prepare": step_prepare, "overlap": step_overlap, "overlap-route": step_overlap_route,
                 "serial": step_serial, "fused": step_fused, "prepare-fused": step_prepare_fused}[args.schedule]
    # one step on a side stream (graph capture wants the work seen once off
    # the capture stream), then the W warm-up steps on the launch stream
    # itself, eager or replayed, so that nothing first-time lands in the
    # timed steps
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        head_step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            head_step()
        torch.cuda.synchronize()
        head_fn = graph.replay
    else:
        head_fn = head_step
    # Clock ramp: the GPU has idled through the host-side setup (the CPU
    # baseline, the uploads), and after a few seconds idle it needs ~15 ms of
    # continuous work before the step reaches its working time (at the
    # prefill shape the first 40 steps ran 0.37-0.41 ms, then 0.349 ms;
    # with 5 warm-up steps the timed block had averaged 0.394 ms against
    # 0.344 ms for the same schedule timed later in the run). So the headline
    # step first repeats, untimed, until RAMP_S seconds have passed; then come
    # the W warm-up steps and the K timed steps.
    t_ramp = time.perf_counter()
    ramp_steps = 0
    while True:
        for _ in range(4):
            head_fn()
        ramp_steps += 4
        torch.cuda.synchronize()
        if time.perf_counter() - t_ramp >= RAMP_S:
            break
    ramp_ms = (time.perf_counter() - t_ramp) * 1000.0
    for _ in range(args.warmup):
        head_fn()
    torch.cuda.synchronize()

    # headline: exactly K steps between two synchronizations
    ms_per_step = timed(head_fn, args.steps)
    head_name = {"prepare": "norm+quant on a second stream beside the dispatch, joined before the combine",
                 "overlap": "norm+quant on a second stream beside dispatch + combine",
                 "overlap-route": "norm+quant on a second stream beside the route",
                 "serial": "serial",
                 "fused": "serial, route and dispatch in one call (moe_route_dispatch)",
                 "prepare-fused": "route, dispatch and norm+quant in one call (moe_route_dispatch_quant), "
                                  "then the combine"}[args.schedule] + \
        (", HIP graph replay" if args.graph else ", eager launches")

    # serial eager pass with per-call events on the launch stream (stage times);
    # each schedule's kernels run once untimed first, so no first launch in
    # the process (its code-object load) falls inside the events
    for warm in (step_serial, step_fused, step_prepare_fused):
        warm()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step_serial(events[i])
    torch.cuda.synchronize()
    # every other schedule gets untimed steps of its own first (its streams'
    # first launches stay out of its figure, as the headline's do)
    serial_ms = timed(step_serial, args.steps)
    # the fused form with per-call events (route + dispatch as one call)
    fused_events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step_fused(fused_events[i])
    torch.cuda.synchronize()
    fused_ms = timed(step_fused, args.steps)
    # route + dispatch + norm + quant in one call, with events
    pf_events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step_prepare_fused(pf_events[i])
    torch.cuda.synchronize()
    prepare_fused_ms = timed(step_prepare_fused, args.steps)
    timed(step_overlap, 5)
    overlap_eager_ms = timed(step_overlap, args.steps)
    timed(step_prepare, 5)
    prepare_eager_ms = timed(step_prepare, args.steps)
    timed(step_overlap_route, 5)
    overlap_route_ms = timed(step_overlap_route, args.steps)

    def graph_ms(step):
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            step()                       # warm the side stream the capture runs on
        stream.wait_stream(side)
        with torch.cuda.graph(g2):
            step()
        torch.cuda.synchronize()
        g2.replay()
        ms = timed(g2.replay, args.steps)
        del g2
        return ms

    overlap_graph_ms = ms_per_step if args.graph and args.schedule == "overlap" else graph_ms(step_overlap)
    serial_graph_ms = ms_per_step if args.graph and args.schedule == "serial" else graph_ms(step_serial)
    fused_graph_ms = ms_per_step if args.graph and args.schedule == "fused" else graph_ms(step_fused)
    prepare_fused_graph_ms = (ms_per_step if args.graph and args.schedule == "prepare-fused"
                              else graph_ms(step_prepare_fused))

    # cold: the 256 MB last-level cache flushed before each step, outside its
    # events, by a 512 MiB write (which leaves up to the cache's size of dirty
    # lines, whose write-back the step then pays) or by a 512 MiB read (which
    # only evicts)
    cold_ms = cold_read_ms = head_cold_ms = head_cold_read_ms = None
    if args.cold_steps > 0:
        flush = torch.empty(1 << 29, dtype=torch.uint8, device=dev)
        flush.fill_(1)

        def cold(step_fn, by_read):
            ce = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.cold_steps)]
            for a, b in ce:
                if by_read:
                    flush.max()
                else:
                    flush.fill_(1)
                a.record(stream)
                step_fn()
                b.record(stream)
            torch.cuda.synchronize()
            return float(np.mean([a.elapsed_time(b) for a, b in ce]))

        cold_ms, cold_read_ms = cold(step_serial, False), cold(step_serial, True)
        head_cold_ms, head_cold_read_ms = cold(head_step, False), cold(head_step, True)
        del flush

    # norm + quant reading the rank-block layout of 8 column shards
    # ([8*T, H/8], what a dim-0 all-gather of the shards leaves)
    rank_block = None
    if H % (8 * 16) == 0:
        tp = 8
        pooled = x.view(T, tp, H // tp).transpose(0, 1).contiguous().view(tp * T, H // tp)
        rb_packed, rb_scales = torch.empty_like(packed), torch.empty_like(scales)
        m.norm_quant_nvfp4_rank_block(pooled, T, qw, w.quant_gain_center, w.eps, gs, packed=rb_packed, scales=rb_scales)
        norm_quant_()
        torch.cuda.synchronize()
        same = bool(torch.equal(rb_packed, packed) and torch.equal(rb_scales, scales))
        re = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in re:
            a.record(stream)
            m.norm_quant_nvfp4_rank_block(pooled, T, qw, w.quant_gain_center, w.eps, gs, packed=rb_packed, scales=rb_scales)
            b.record(stream)
        torch.cuda.synchronize()
        rb_ms = float(np.mean([a.elapsed_time(b) for a, b in re]))
        rank_block = {"tp": tp, "ms": round(rb_ms, 4), "same_bytes_as_contiguous": same}
        del pooled, rb_packed, rb_scales

    fc1 = fc1_swiglu = None
    if args.fc1:
        fc1 = time_expert_fc1(m, wl, torch, dev, stream)
        fc1_swiglu = time_expert_fc1(m, wl, torch, dev, stream, swiglu=True)
        # the other token counts the act-fusion GEMM page times the FC1 at
        fc1["other_token_counts"] = {}
        for tok in (8192, 65536):
            r = time_expert_fc1(m, wl, torch, dev, stream, tokens=tok)
            fc1["other_token_counts"][str(tok)] = {k_: r[k_] for k_ in ("ms", "TFLOPs", "frac_of_fp16_mfma_peak")}
            torch.cuda.empty_cache()

    names = ["route", "dispatch", "norm_quant", "combine"]
    stage_ms = {n: float(np.mean([events[i][j].elapsed_time(events[i][j + 1]) for i in range(args.steps)]))
                for j, n in enumerate(names)}
    valid_slots = int(offsets[-1].item())
    nbytes = algorithmic_bytes(w, hidden.element_size(), valid_slots)
    total_bytes = sum(nbytes.values())
    stages = {n: {"ms": round(stage_ms[n], 4), "bytes": nbytes[n],
                  "GBps": round(nbytes[n] / (stage_ms[n] * 1e-3) / 1e9, 1)} for n in names}
    # per-step spread of the serial pass (first call's start to last call's end)
    step_ev = np.array([events[i][0].elapsed_time(events[i][4]) for i in range(args.steps)])
    serial_spread = {"p10_ms": round(float(np.percentile(step_ev, 10)), 4),
                     "median_ms": round(float(np.median(step_ev)), 4),
                     "p90_ms": round(float(np.percentile(step_ev, 90)), 4)}
    proj_flop = 2.0 * T * H * E
    if rank_block is not None:
        rank_block["GBps"] = round(nbytes["norm_quant"] / (rank_block["ms"] * 1e-3) / 1e9, 1)
        stages["norm_quant_rank_block"] = rank_block
    stages["route"]["proj_TFLOPs_fp32_equiv"] = round(proj_flop / (stage_ms["route"] * 1e-3) / 1e12, 2)
    rd_ms = float(np.mean([fused_events[i][0].elapsed_time(fused_events[i][1]) for i in range(args.steps)]))
    rd_bytes = nbytes["route"] + nbytes["dispatch"]
    stages["route_dispatch"] = {"ms": round(rd_ms, 4), "bytes": rd_bytes,
                                "GBps": round(rd_bytes / (rd_ms * 1e-3) / 1e9, 1),
                                "note": "moe_route_dispatch: the fused call, from the fused pass"}
    rdq_ms = float(np.mean([pf_events[i][0].elapsed_time(pf_events[i][1]) for i in range(args.steps)]))
    rdq_bytes = rd_bytes + nbytes["norm_quant"]
    stages["route_dispatch_quant"] = {"ms": round(rdq_ms, 4), "bytes": rdq_bytes,
                                      "GBps": round(rdq_bytes / (rdq_ms * 1e-3) / 1e9, 1),
                                      "note": "moe_route_dispatch_quant: route, dispatch and norm + quant in "
                                              "one call, from its own pass"}

    comb_gbs = nbytes["combine"] / (stage_ms["combine"] * 1e-3) / 1e9
    tokens_per_s = T / (ms_per_step * 1e-3)
    hbm_gbs = total_bytes / (ms_per_step * 1e-3) / 1e9

    # Reference point for the HBM-bound kernels: a plain 1 GiB elementwise
    # copy (torch.neg on int16: 1 GiB read + 1 GiB written), timed on its own.
    copy_gbs = None
    if args.copy_calib or args.copy_ref:
        ca = torch.zeros(1 << 29, dtype=torch.int16, device=dev)
        cb = torch.empty_like(ca)
        torch.neg(ca, out=cb)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        reps = 5
        for _ in range(reps):
            torch.neg(ca, out=cb)
        e1.record(stream)
        torch.cuda.synchronize()
        copy_gbs = 2.0 * (1 << 30) * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del ca, cb

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "clock_ramp": {"untimed_steps": ramp_steps, "ms": round(ramp_ms, 1),
                       "note": "the headline step repeated untimed before the warm-up steps, so the GPU "
                               "leaves its idle clock before the timed region"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic (seeded numpy PCG64; BF16 storage, FP32 arithmetic, BF16x3 MFMA projection)",
        "config": {"workload": "%s: T=%d H=%d E=%d k=%d, %d%% invalid tokens" % (
            w.name, T, H, E, k, round(100 * w.invalid_token_frac)),
            "tokens": T, "hidden": H, "experts": E, "top_k": k, "valid_tokens": int(mask_np.sum())},
        "hbm_GBps_algorithmic": round(hbm_gbs, 1),
        "hbm_frac_of_peak": round(hbm_gbs / HBM_PEAK_GBS, 4),
        "valid_tokens_per_s": round(int(mask_np.sum()) / (ms_per_step * 1e-3), 1),
        "stages": stages,
        "expert_fc1": fc1,
        "expert_fc1_swiglu": fc1_swiglu,
        "schedules": {"headline": head_name, "headline_ms": round(ms_per_step, 4),
                      "serial_eager_ms": round(serial_ms, 4), "fused_eager_ms": round(fused_ms, 4),
                      "fused_graph_ms": round(fused_graph_ms, 4),
                      "prepare_fused_eager_ms": round(prepare_fused_ms, 4),
                      "prepare_fused_graph_ms": round(prepare_fused_graph_ms, 4),
                      "prepare_eager_ms": round(prepare_eager_ms, 4),
                      "overlap_eager_ms": round(overlap_eager_ms, 4),
                      "overlap_route_eager_ms": round(overlap_route_ms, 4),
                      "overlap_graph_ms": round(overlap_graph_ms, 4),
                      "serial_graph_ms": round(serial_graph_ms, 4),
                      "serial_cold_ms": None if cold_ms is None else round(cold_ms, 4),
                      "serial_cold_read_flush_ms": None if cold_read_ms is None else round(cold_read_ms, 4),
                      "headline_cold_ms": None if head_cold_ms is None else round(head_cold_ms, 4),
                      "headline_cold_read_flush_ms": None if head_cold_read_ms is None else round(head_cold_read_ms, 4),
                      "serial_steps": serial_spread},
        "device_copy_GBps": None if copy_gbs is None else round(copy_gbs, 1),
        "hbm_frac_of_device_copy": None if copy_gbs is None else round(hbm_gbs / copy_gbs, 4),
        "roofline": {"kernel": "combine", "bound": "hbm", "achieved": round(comb_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(comb_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(w.name)},
        "cpu_baseline": None,
    }
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result))


if __name__ == "__main__":
    main()
