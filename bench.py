#!/usr/bin/env python3
"""Benchmark of the MoE FFN forward (routing + grouped expert GEMMs + combine)
on one MI355X.

One step = moe_route + moe_forward over one batch whose inputs already sit in
HBM.  The headline line is the large-T bf16 prefill layer (T=8192, H=2048,
I=768, E=128, top-8, Zipf-skewed routing): value = tokens/s.  The same JSON
line carries
  * roofline: the dominant kernel (the grouped Gate/Up GEMM), its algorithmic
    flops per launch over its average duration, measured with HIP events the
    library records on its own stream during the timed steps;
  * decode: µs/layer at B=1..4 (bf16 route-direct path, H=2048 I=768 E=128),
    cold HBM (a 1 GiB buffer is read between iterations, so no expert weight
    is left in the L2s or the MALL), with the HBM fraction of its dominant kernel;
  * fp8: the FP8 per-tensor decode (B=1..4, H=4096 I=192 E=192) and the FP8
    128x128-blockwise prefill (T=4096, H=4096, I=512) -- skipped with --quick;
  * backward_fp8_mx32: the MX training backward at the MX prefill shape
    (per-stage times against their bounds);
  * cpu_baseline: the CPU oracle on a bounded sample of the headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s (large T) + µs/layer at B=1-4; % of HBM BW / MFMA peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def dev_inputs(torch, a, wl):
    x = torch.from_numpy(a["x"].view(np.int16)).cuda().view(torch.bfloat16)
    lg = torch.from_numpy(a["logits"]).cuda()
    return x, lg


def dev_weights(torch, moe, w, quant):
    if quant == "bf16":
        gu = torch.from_numpy(w["w_gate_up"].view(np.int16)).cuda()
        dn = torch.from_numpy(w["w_down"].view(np.int16)).cuda()
        scales = None
    else:
        gu = torch.from_numpy(w["w_gate_up"]).cuda()
        dn = torch.from_numpy(w["w_down"]).cuda()
        scales = (torch.from_numpy(w["s_gate_up"]).cuda(), torch.from_numpy(w["s_down"]).cuda())
        if quant == "fp8_mx32":
            scales = moe.pack_mx_scales(*scales)
    pw = moe.pack_weights(gu, dn, quant)
    torch.cuda.synchronize()
    del gu, dn
    return pw, scales


class Layer:
    """Preallocated routes, output and workspaces for repeated steps."""

    def __init__(self, torch, moe, wl, T, x, lg, weights, path="auto"):
        self.torch, self.moe, self.wl, self.T = torch, moe, wl, T
        self.x, self.lg = x, lg
        self.pw, self.scales = weights
        self.path = moe.select_path(T, wl.H, wl.I, wl.E, wl.k, wl.quant, path)
        self.routes = moe.Routes(T, wl.E, wl.k, x.device)
        self.out = torch.empty((T, wl.H), dtype=torch.bfloat16, device=x.device)
        n = moe.forward_workspace_size(T, wl.H, wl.I, wl.E, wl.k, wl.quant, self.path)
        self.ws = torch.empty(max(n, 256), dtype=torch.uint8, device=x.device)
        rn = moe.route_workspace_size(T, wl.E, wl.k)
        self.rws = torch.empty(rn, dtype=torch.uint8, device=x.device) if rn else None

    def step(self, events=None, lg=None):
        self.moe.route(self.lg if lg is None else lg, self.wl.k, out=self.routes, workspace=self.rws)
        return self.moe.forward(self.x, self.routes, self.pw, quant=self.wl.quant,
                                scales=self.scales, out=self.out, path=self.path, workspace=self.ws,
                                events=events)


def stage_times(torch, ev_sets, names):
    """Average ms per stage over the recorded steps."""
    n = len(names)
    tot = np.zeros(n)
    for evs in ev_sets:
        for i in range(n):
            tot[i] += evs[i].elapsed_time(evs[i + 1])
    return {names[i]: tot[i] / len(ev_sets) for i in range(n)}


def bench_prefill(torch, moe, name, steps, warmup, stage_steps=10):
    """Prefill throughput: `steps` timed steps (moe_route + moe_forward) whose only
    instrumentation is the pair of HIP events around the Gate/Up launch (the
    roofline kernel; every recorded event costs the stream a few microseconds),
    then `stage_steps` untimed steps with events between all stages for the
    per-stage breakdown."""
    from workloads import WORKLOADS, workload_inputs, workload_weights
    wl = WORKLOADS[name]
    a = workload_inputs(name)
    w = workload_weights(name)
    x, lg = dev_inputs(torch, a, wl)
    layer = Layer(torch, moe, wl, wl.T, x, lg, dev_weights(torch, moe, w, wl.quant))
    for _ in range(warmup):
        layer.step()
    _, names = layer.step(events=[torch.cuda.Event(enable_timing=True) for _ in range(8)])
    g = names.index("gate_up")
    torch.cuda.synchronize()
    gu_pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in gu_pairs:                   # create the events before the timed region
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in gu_pairs:
        evs = [None] * (len(names) + 1)
        evs[g], evs[g + 1] = e0, e1
        layer.step(events=evs)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    gate_up_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in gu_pairs]))
    ev_sets = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(stage_steps)]
    for evs in ev_sets:
        layer.step(events=evs)
    torch.cuda.synchronize()
    st = stage_times(torch, ev_sets, names)
    counts = layer.routes.expert_counts.cpu().numpy()
    return dict(wl=wl, dt=dt, stages_ms=st, gate_up_ms=gate_up_ms, path=layer.path, counts=counts,
                layer=layer, host=(a, w))


# HBM traffic of one Gate/Up launch from two rocprofv3 counter passes (FETCH_SIZE,
# WRITE_SIZE; KiB per dispatch, median over the run's launches), each scaled by
# what the counter reads for a plain 1 GiB copy kernel in the same run:
# FETCH_SIZE reads 524300.5 KiB for 1 GiB read (x2.0), WRITE_SIZE exactly 1 GiB
# (x1.0).  Valid only for the GEMM source the counters were taken on; any edit
# to it turns the figure into null.
FETCH_SCALE, WRITE_SCALE = 1048576.0 / 524300.5, 1.0
_GEMM_SHA = "f152d3404fb11001f3fd989a2db6f296e23cc0bd32c76b4281ca7cc08aba7230"
COUNTER_TRAFFIC = {
    "prefill_bf16": dict(gemm_sha256=_GEMM_SHA, fetch_kib=803991.4, write_kib=98324.4),
    "prefill_fp8_block": dict(gemm_sha256=_GEMM_SHA, fetch_kib=382525.1, write_kib=17436.9),
    "prefill_fp8_mx": dict(gemm_sha256=_GEMM_SHA, fetch_kib=421981.3, write_kib=17499.5),
}


def counter_traffic(name):
    import hashlib
    rec = COUNTER_TRAFFIC.get(name)
    if rec is None:
        return None
    src = os.path.join(ROOT, "routing_grouped_expert_index_amd", "csrc", "gemm.hip")
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec["gemm_sha256"]:
            return None
    return round((rec["fetch_kib"] * FETCH_SCALE + rec["write_kib"] * WRITE_SCALE) * 1024.0)


def bench_backward(torch, moe, steps, warmup, stage_steps=10):
    """The MX training backward (moe_backward) at the MX prefill layer's shape,
    and the training step around it (weight preparation + MX forward from it):
    seeded bf16 master weights, x, logits and upstream gradient; the routing and
    the weight preparation run once, outside the timed region.  Timed: `steps`
    calls between two HIP events on the stream; then `stage_steps` calls with
    events on every stage for the breakdown, each stage priced against its
    bound (the products against the fp8 MFMA peak, the weight-gradient kernels
    -- fp32 outputs, each written once -- against HBM)."""
    from workloads import WORKLOADS, random_activations, random_upstream, random_weights
    wl = WORKLOADS["prefill_fp8_mx"]
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    R = T * k
    a = random_activations(T, H, E, seed=wl.act_seed)
    w = random_weights(E, H, I, "bf16", seed=wl.weight_seed)
    dout = random_upstream(T, H, seed=wl.act_seed)
    dev = torch.device("cuda:0")
    b16 = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
    x, d = b16(a["x"]), b16(dout)
    routes = moe.route(torch.from_numpy(a["logits"]).to(dev), k)
    wgu, wd = b16(w["w_gate_up"]), b16(w["w_down"])
    tw = moe.prepare_mx_train_weights(wgu, wd)   # (the first call loads the kernels)
    torch.cuda.synchronize()
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record()
    tw = moe.prepare_mx_train_weights(wgu, wd)
    p1.record()
    torch.cuda.synchronize()
    prep_ms = p0.elapsed_time(p1)
    del wgu, wd
    out = {"dx": torch.empty((T, H), dtype=torch.bfloat16, device=dev),
           "dgate": torch.empty((T, k), dtype=torch.float32, device=dev),
           "dw_gate_up": torch.empty((E, H, 2 * I), dtype=torch.bfloat16, device=dev),
           "dw_down": torch.empty((E, I, H), dtype=torch.bfloat16, device=dev)}
    ws = torch.empty(moe.backward_workspace_size(T, H, I, E, k), dtype=torch.uint8, device=dev)
    for _ in range(warmup):
        moe.backward(x, routes, tw, d, workspace=ws, out=out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        moe.backward(x, routes, tw, d, workspace=ws, out=out)
    e1.record()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / steps
    # the MX forward from the same preparation (the training step's forward)
    fout = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    fws = torch.empty(moe.forward_workspace_size(T, H, I, E, k, "fp8_mx32", "grouped"), dtype=torch.uint8, device=dev)
    for _ in range(3):
        moe.forward(x, routes, tw.forward, quant="fp8_mx32", scales=tw.forward_scales, out=fout, path="grouped",
                    workspace=fws)
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record()
    for _ in range(steps):
        moe.forward(x, routes, tw.forward, quant="fp8_mx32", scales=tw.forward_scales, out=fout, path="grouped",
                    workspace=fws)
    f1.record()
    torch.cuda.synchronize()
    fwd_ms = f0.elapsed_time(f1) / steps
    del fout, fws
    ev_sets = [[torch.cuda.Event(enable_timing=True) for _ in range(14)] for _ in range(stage_steps)]
    names = None
    for evs in ev_sets:
        _, names = moe.backward(x, routes, tw, d, workspace=ws, out=out, events=evs)
    torch.cuda.synchronize()
    st = stage_times(torch, ev_sets, names)
    counts = routes.expert_counts.cpu().numpy()
    Rp = int(np.sum((counts + 63) // 64 * 64))           # padded route positions of the weight gradients
    flops = {"gate_up": 2.0 * R * H * 2 * I, "down": 2.0 * R * I * H, "dh": 2.0 * R * H * I,
             "dx_rows": 2.0 * R * 2 * I * H}
    wbytes = {"wgrad_gate_up": 2.0 * E * H * 2 * I + (H + 2 * I) * Rp * (1 + 1 / 32),
              "wgrad_down": 2.0 * E * I * H + (I + H) * Rp * (1 + 1 / 32)}
    stages = {}
    for n, ms in st.items():
        rec = dict(us=round(ms * 1e3, 2))
        if n in flops:
            tf = flops[n] / (ms / 1e3) / 1e12
            rec.update(bound="mfma", achieved=round(tf, 1), unit="TFLOP/s", frac=round(tf / PEAK_FP8_TFLOPS, 4))
        elif n in wbytes:
            gbs = wbytes[n] / (ms / 1e3) / 1e9
            rec.update(bound="hbm", achieved=round(gbs, 1), unit="GB/s", frac=round(gbs / PEAK_HBM_GBS, 4),
                       bytes_per_launch=int(wbytes[n]))
        stages[n] = rec
    dom = max(stages, key=lambda n: stages[n]["us"])
    del out, ws, tw
    return dict(workload="MX training backward at prefill_fp8_mx: T=4096 H=4096 I=512 E=128 top-8; bf16 master "
                         "weights, dW in bf16",
                tokens_per_s=round(T * steps / dt, 1), ms_per_step=round(step_ms, 4),
                ms_per_step_wall=round(dt / steps * 1e3, 4), prepare_weights_ms=round(prep_ms, 3),
                forward_ms=round(fwd_ms, 4),
                train_step_ms=round(prep_ms + fwd_ms + step_ms, 4),
                stages=stages, dominant=dict(stage=dom, **stages[dom]),
                flops_per_step=18.0 * R * H * I, padded_routes=Rp)


def roofline_gemm(wl, gate_up_ms, peak):
    R = wl.T * wl.k
    flops = 4.0 * R * wl.H * wl.I            # Gate/Up: 2 flops x R rows x H x 2I
    t = gate_up_ms / 1e3
    achieved = flops / t / 1e12
    return dict(kernel="grouped_gemm_kernel (Gate/Up + SwiGLU)", bound="mfma", achieved=round(achieved, 2),
                peak=peak, unit="TFLOP/s", frac=round(achieved / peak, 4),
                traffic=counter_traffic(wl.name), traffic_unit="bytes per launch",
                flops_per_launch=flops, avg_launch_us=round(gate_up_ms * 1e3, 2))


def bench_decode(torch, moe, name, batches, iters, nsets=32):
    """Cold-HBM decode latency of one layer (moe_route + moe_forward), 32 rotating
    routing sets, a 1 GiB read before each iteration.  Three timings per batch:
    stream launches bracketed by two HIP events; the same step captured once in
    a HIP graph and replayed; and a run with events between the stages for the
    dominant kernel's own duration."""
    from workloads import WORKLOADS, random_activations, workload_weights
    wl = WORKLOADS[name]
    w = workload_weights(name)
    weights = dev_weights(torch, moe, w, wl.quant)
    # eviction by READING 1 GiB (more than the 256 MB MALL and the L2s): a written
    # eviction buffer leaves dirty lines whose write-back would compete with the
    # layer's reads and halve the measured bandwidth
    evict = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    elem = 2 if wl.quant == "bf16" else 1
    res = {}
    for B in batches:
        sets = [random_activations(B, wl.H, wl.E, 10000 + i) for i in range(nsets)]
        xs = [dev_inputs(torch, s, wl) for s in sets]
        layer = Layer(torch, moe, wl, B, xs[0][0].clone(), xs[0][1].clone(), weights)

        def load(it):
            layer.x.copy_(xs[it % nsets][0])
            layer.lg.copy_(xs[it % nsets][1])

        def timed(run):
            ts = []
            for it in range(iters + 2):
                load(it)
                evict.amax()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                run()
                e1.record()
                if it >= 2:
                    ts.append((e0, e1))
            torch.cuda.synchronize()
            return float(np.median([a.elapsed_time(b) for a, b in ts])) * 1e3   # us

        # route and forward separately: one event between the two calls
        tr, tf = [], []
        for it in range(iters + 2):
            load(it)
            evict.amax()
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            e0.record()
            moe.route(layer.lg, wl.k, out=layer.routes, workspace=layer.rws)
            e1.record()
            moe.forward(layer.x, layer.routes, layer.pw, quant=wl.quant, scales=layer.scales,
                        out=layer.out, path=layer.path, workspace=layer.ws)
            e2.record()
            if it >= 2:
                tr.append((e0, e1))
                tf.append((e1, e2))
        torch.cuda.synchronize()
        t_route_only = float(np.median([a.elapsed_time(b) for a, b in tr])) * 1e3
        t_fwd_only = float(np.median([a.elapsed_time(b) for a, b in tf])) * 1e3
        # the forward's device span: events attached to its first and last kernel
        # dispatches (moe_forward_timed), the figure a kernel trace reports
        td = []
        for it in range(iters + 2):
            load(it)
            evict.amax()
            moe.route(layer.lg, wl.k, out=layer.routes, workspace=layer.rws)
            d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            moe.forward(layer.x, layer.routes, layer.pw, quant=wl.quant, scales=layer.scales, out=layer.out,
                        path=layer.path, workspace=layer.ws, device_events=(d0, d1))
            if it >= 2:
                td.append((d0, d1))
        torch.cuda.synchronize()
        t_fwd_dev = float(np.median([a.elapsed_time(b) for a, b in td])) * 1e3
        t_fwd = timed(layer.step)
        # the routing folded into the first kernel (moe_decode_forward), route-direct only
        t_fused = None
        if layer.path == "route_direct":
            t_fused = timed(lambda: moe.decode_forward(layer.lg, layer.x, wl.k, layer.pw, quant=wl.quant,
                                                       scales=layer.scales, out=layer.out, routes=layer.routes,
                                                       path=layer.path, workspace=layer.ws))
        # the step captured once (as a serving loop would) and replayed
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            layer.step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer.step()
        t_graph = timed(g.replay)
        # warm: the captured step replayed back to back, weights left in the caches
        nwarm = 200
        for _ in range(10):
            g.replay()
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0.record()
        for _ in range(nwarm):
            g.replay()
        w1.record()
        torch.cuda.synchronize()
        t_graph_warm = w0.elapsed_time(w1) / nwarm * 1e3
        del g
        # stage events: the dominant kernel's duration
        ev_sets = []
        for it in range(iters + 2):
            load(it)
            evict.amax()
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
            for e in evs:
                e.record()
            _, names = layer.step(events=evs)
            if it >= 2:
                ev_sets.append((evs, names))
        torch.cuda.synchronize()
        distinct = []
        for it in range(nsets):
            ids = moe.route(xs[it][1], wl.k).topk_ids.cpu().numpy()
            distinct.append(len(np.unique(ids)))
        dom = []
        for evs, names in ev_sets:
            dname = "rd_gate_up" if "rd_gate_up" in names else "gate_up"
            i = names.index(dname)
            dom.append(evs[i].elapsed_time(evs[i + 1]))
        t_dom = float(np.median(dom)) * 1e3
        D = float(np.mean(distinct))
        w_bytes = D * 3 * wl.H * wl.I * elem
        dom_bytes = D * 2 * wl.H * wl.I * elem + B * wl.H * elem   # Gate/Up weights + activations
        res[B] = dict(us_per_layer=round(t_fwd, 2),
                      us_per_layer_fused=None if t_fused is None else round(t_fused, 2),
                      us_route=round(t_route_only, 2),
                      us_forward=round(t_fwd_only, 2), us_per_layer_graph=round(t_graph, 2),
                      us_per_layer_graph_warm=round(t_graph_warm, 2),
                      tokens_per_s=round(B / (t_fwd * 1e-6), 1),
                      path=layer.path, distinct_experts=round(D, 2),
                      us_forward_device=round(t_fwd_dev, 2),
                      hbm_frac_forward=round(w_bytes / (t_fwd_only * 1e-6) / (PEAK_HBM_GBS * 1e9), 4),
                      hbm_frac_forward_device=round(w_bytes / (t_fwd_dev * 1e-6) / (PEAK_HBM_GBS * 1e9), 4),
                      hbm_frac_layer=round(w_bytes / (t_fwd * 1e-6) / (PEAK_HBM_GBS * 1e9), 4),
                      hbm_frac_layer_graph=round(w_bytes / (t_graph * 1e-6) / (PEAK_HBM_GBS * 1e9), 4),
                      dominant=dict(kernel=dname, bound="hbm", avg_launch_us=round(t_dom, 2),
                                    achieved=round(dom_bytes / (t_dom * 1e-6) / 1e9, 1),
                                    peak=PEAK_HBM_GBS, unit="GB/s",
                                    frac=round(dom_bytes / (t_dom * 1e-6) / (PEAK_HBM_GBS * 1e9), 4)))
        log(f"decode {name} B={B}: {t_fwd:.2f} us/layer, fused {t_fused} (route {t_route_only:.2f} + forward "
            f"{t_fwd_only:.2f}, forward device span {t_fwd_dev:.2f}; "
            f"graph {t_graph:.2f}, warm graph {t_graph_warm:.2f}), "
            f"{res[B]['dominant']['kernel']} {t_dom:.2f} us {res[B]['dominant']['achieved']} GB/s")
    del evict
    return res


def bench_router(torch, moe, batches, iters, H=2048, E=128, k=8):
    """Cold-HBM latency of the router scores x W_r plus routing in one call
    (moe_route_project, W_r fp32 [H, E]) against the two-call alternative
    (torch's fp32 product, then moe_route) and moe_route alone on given logits."""
    from workloads import random_activations
    evict = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    res = {}
    for B in batches:
        a = random_activations(B, H, E, 500 + B, logits="router")
        x = torch.from_numpy(a["x"].view(np.int16)).cuda().view(torch.bfloat16)
        wr = torch.from_numpy(a["w_router"]).cuda()
        routes = moe.Routes(B, E, k, x.device)
        lg = torch.empty((B, E), dtype=torch.float32, device=x.device)
        ws = torch.zeros(moe.route_project_workspace_size(B, H, E, k), dtype=torch.uint8, device=x.device)
        rws_n = moe.route_workspace_size(B, E, k)
        rws = torch.empty(rws_n, dtype=torch.uint8, device=x.device) if rws_n else None

        def fused():
            moe.route_project(x, wr, k, out=routes, logits=lg, workspace=ws)

        def two_calls():
            torch.matmul(x.float(), wr, out=lg)
            moe.route(lg, k, out=routes, workspace=rws)

        def route_only():
            moe.route(lg, k, out=routes, workspace=rws)

        def timed(run):
            ts = []
            for it in range(iters + 2):
                evict.amax()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                run()
                e1.record()
                if it >= 2:
                    ts.append((e0, e1))
            torch.cuda.synchronize()
            return float(np.median([p.elapsed_time(q) for p, q in ts])) * 1e3

        t_f, t_2, t_r = timed(fused), timed(two_calls), timed(route_only)
        nbytes = H * E * 4 + B * H * 2
        res[B] = dict(us_route_project=round(t_f, 2), us_matmul_then_route=round(t_2, 2),
                      us_route_only=round(t_r, 2), bytes=nbytes,
                      achieved_gbs=round(nbytes / (t_f * 1e-6) / 1e9, 1))
        log(f"router B={B}: route_project {t_f:.2f} us, matmul + route {t_2:.2f} us, route alone {t_r:.2f} us")
    del evict
    return res


# The route-direct latencies printed by "perf: add small-batch route MMA for MoE"
# (Performance tables, forced route path, single-op CUDA graph with preallocated
# output, top-8, on an H20): context for the same shapes here, not a target.
PAGES_ROUTE_US = {
    "fp8_per_tensor E=192 H=4096 I=192": [13.243, 16.833, 22.773, 30.663, 35.983, 41.554, 47.259, 54.124],
    "fp8_block128 E=128 H=2048 I=768": [17.349, 29.863, 40.708, 52.732, 62.510, 73.040, 84.419, 94.352],
    "fp8_block128 E=128 H=4096 I=512": [19.779, 37.585, 52.295, 63.833, 85.218, 98.465, 111.362, 121.922],
}


def bench_pages_shapes(torch, moe, iters, batches=range(1, 9)):
    """moe_forward alone (routes given, as the pages time their op) captured in a
    HIP graph with preallocated output, at the pages' three FP8 decode shapes:
    replayed cold (a 1 GiB read before each replay) and warm (back to back), and
    launched straight on the stream, cold and warm (each call between two events)."""
    from workloads import random_activations, random_weights, workload_weights
    evict = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    shapes = [("fp8_per_tensor E=192 H=4096 I=192", 192, 4096, 192, "fp8_per_tensor",
               lambda: workload_weights("decode_fp8_tensor")),
              ("fp8_block128 E=128 H=2048 I=768", 128, 2048, 768, "fp8_block128",
               lambda: random_weights(128, 2048, 768, "fp8_block128", 6)),
              ("fp8_block128 E=128 H=4096 I=512", 128, 4096, 512, "fp8_block128",
               lambda: workload_weights("prefill_fp8_block"))]
    # leave the idle clock state before the first timing (tens of milliseconds of load)
    for _ in range(200):
        evict.amax()
    torch.cuda.synchronize()
    res = {}
    for key, E, H, I, quant, wfn in shapes:
        pw, scales = dev_weights(torch, moe, wfn(), quant)
        out_k = {}
        for B in batches:
            a = random_activations(B, H, E, 20000 + B)
            x = torch.from_numpy(a["x"].view(np.int16)).cuda().view(torch.bfloat16)
            r = moe.route(torch.from_numpy(a["logits"]).cuda(), 8)
            out = torch.empty((B, H), dtype=torch.bfloat16, device="cuda")
            path = moe.select_path(B, H, I, E, 8, quant)
            ws = torch.empty(max(256, moe.forward_workspace_size(B, H, I, E, 8, quant, path)),
                             dtype=torch.uint8, device="cuda")

            def fwd():
                moe.forward(x, r, pw, quant=quant, scales=scales, out=out, path=path, workspace=ws)

            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                fwd()
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fwd()
            def cold_median(run, cold=True):
                ts = []
                for it in range(iters + 2):
                    if cold:
                        evict.amax()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    run()
                    e1.record()
                    if it >= 2:
                        ts.append((e0, e1))
                torch.cuda.synchronize()
                return float(np.median([p.elapsed_time(q) for p, q in ts])) * 1e3

            cold = cold_median(g.replay)
            cold_stream = cold_median(fwd)   # the same launches straight on the stream
            # stream, warm: no read between the calls, so the weights stay in the caches;
            # each call timed between its own two events (the device time of its launches)
            warm_stream = cold_median(fwd, cold=False)
            for _ in range(20):
                g.replay()
            w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            nwarm = 200
            w0.record()
            for _ in range(nwarm):
                g.replay()
            w1.record()
            torch.cuda.synchronize()
            warm = w0.elapsed_time(w1) / nwarm * 1e3
            del g
            h20 = PAGES_ROUTE_US[key][B - 1]
            out_k[B] = dict(path=path, us_graph_cold=round(cold, 2), us_graph_warm=round(warm, 2),
                            us_stream_cold=round(cold_stream, 2), us_stream_warm=round(warm_stream, 2),
                            pages_h20_us=h20, h20_over_stream_warm=round(h20 / warm_stream, 3),
                            h20_over_warm=round(h20 / warm, 3), h20_over_cold=round(h20 / cold, 3),
                            h20_over_stream_cold=round(h20 / cold_stream, 3))
            log(f"{key} B={B} ({path}): graph cold {cold:.2f} us, warm {warm:.2f} us, stream cold "
                f"{cold_stream:.2f} us, stream warm {warm_stream:.2f} us (pages, H20: {h20} us)")
        res[key] = out_k
        del pw, scales
        torch.cuda.empty_cache()
    del evict
    return res


def layer_fractions(wl, t_step, peak_tflops):
    """The whole step against the dense MFMA peak and against HBM: algorithmic flops
    6*R*H*I; the HBM floor with the gather fused = every expert's weights once, x
    once (FP8: and its quantised copy written and read), h and y written and read
    once, out written once."""
    R = wl.T * wl.k
    elem_w = 2 if wl.quant == "bf16" else 1
    flops = 6.0 * R * wl.H * wl.I
    h_b = 2 if wl.quant == "bf16" else 1
    bytes_floor = (wl.E * 3 * wl.H * wl.I * elem_w + wl.T * wl.H * 2 + 2 * R * wl.I * h_b
                   + 2 * R * wl.H * 2 + wl.T * wl.H * 2)
    if wl.quant != "bf16":
        bytes_floor += 2 * wl.T * wl.H        # the quantised x, written and read once
    mf = flops / t_step / (peak_tflops * 1e12)
    hf = bytes_floor / t_step / (PEAK_HBM_GBS * 1e9)
    return dict(flops=flops, bytes_floor=bytes_floor, mfma_frac=round(mf, 4), hbm_frac=round(hf, 4),
                bound_frac=round(max(mf, hf), 4), us_per_step=round(t_step * 1e6, 2))


def bench_crossover(torch, moe, name, batches, iters, nsets=16):
    """Cold route+forward latency with the path forced each way, for the dispatch rule."""
    from workloads import WORKLOADS, random_activations, workload_weights
    wl = WORKLOADS[name]
    weights = dev_weights(torch, moe, workload_weights(name), wl.quant)
    evict = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    res = {}
    for B in batches:
        xs = [dev_inputs(torch, random_activations(B, wl.H, wl.E, 10000 + i), wl) for i in range(nsets)]
        row = {}
        for path in ("grouped", "route_direct"):
            layer = Layer(torch, moe, wl, B, xs[0][0].clone(), xs[0][1].clone(), weights, path=path)
            ts = []
            for it in range(iters + 2):
                layer.x.copy_(xs[it % nsets][0])
                layer.lg.copy_(xs[it % nsets][1])
                evict.amax()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                layer.step()
                e1.record()
                if it >= 2:
                    ts.append((e0, e1))
            torch.cuda.synchronize()
            row[path] = round(float(np.median([a.elapsed_time(b) for a, b in ts])) * 1e3, 2)
        row["auto"] = moe.select_path(B, wl.H, wl.I, wl.E, wl.k, wl.quant, "auto")
        res[B] = row
        log(f"crossover {name} B={B}: grouped {row['grouped']} us, route_direct {row['route_direct']} us, "
            f"auto takes {row['auto']}")
    del evict
    return res


def cpu_baseline(a, w, wl, budget_s=15.0):
    import oracle
    lg, x = a["logits"], a["x"]
    t0 = time.perf_counter()
    r = oracle.route(lg, wl.k)
    oracle.forward(x, r["topk_ids"], r["topk_weights"], w["w_gate_up"], w["w_down"], quant=wl.quant,
                   s_gate_up=w["s_gate_up"], s_down=w["s_down"], tokens=np.arange(32, dtype=np.int32))
    probe = time.perf_counter() - t0
    n = int(min(wl.T, max(64, 32 * budget_s / max(probe, 1e-3))))
    tok = np.arange(n, dtype=np.int32)
    t0 = time.perf_counter()
    r = oracle.route(lg, wl.k)
    oracle.forward(x, r["topk_ids"], r["topk_weights"], w["w_gate_up"], w["w_down"], quant=wl.quant,
                   s_gate_up=w["s_gate_up"], s_down=w["s_down"], tokens=tok)
    dt = time.perf_counter() - t0
    return dict(value=round(n / dt, 2), unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"routing of all {wl.T} tokens + layer output of the first {n} tokens "
                       f"of {wl.name} (fp64 C oracle, gcc -O3 -fopenmp without -march=native so the library "
                       f"runs on any x86-64 host; no tuning), {dt:.1f} s")


def profile_only(torch, moe, args):
    """Short runs of single workloads for rocprofv3 counter passes."""
    for name in args.only.split(","):
        if name == "copy":
            # a plain copy kernel of known size (1 GiB read + 1 GiB written per launch):
            # the reference that scales the FETCH_SIZE / WRITE_SIZE counters
            src = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
            dst = torch.empty_like(src)
            for _ in range(args.steps):
                torch.mul(src, 1, out=dst)
            torch.cuda.synchronize()
            log(f"copy: {args.steps} x 1 GiB elementwise copy kernels")
        elif name == "pages_shapes":
            bench_pages_shapes(torch, moe, args.decode_iters)
        elif name == "router":
            bench_router(torch, moe, (1, 2, 3, 4), args.decode_iters)
        elif name.startswith("crossover_"):
            bench_crossover(torch, moe, name[len("crossover_"):], range(1, 17), 30)
        elif name == "backward_fp8_mx":
            bw = bench_backward(torch, moe, args.steps, args.warmup)
            log(f"{name}: {bw['ms_per_step']:.3f} ms/step, stages us { {k: v['us'] for k, v in bw['stages'].items()} }")
        elif name.startswith("prefill"):
            pf = bench_prefill(torch, moe, name, args.steps, args.warmup)
            log(f"{name}: {pf['dt'] / args.steps * 1e3:.3f} ms/step, stages us "
                f"{ {k: round(float(v) * 1e3, 1) for k, v in pf['stages_ms'].items()} }")
            del pf
        else:
            res = bench_decode(torch, moe, name, (1, 2, 3, 4), args.decode_iters)
            log(f"{name}: { {b: r['us_per_layer'] for b, r in res.items()} }")
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the part leaves its idle clock state only after a few tens of milliseconds of
    # load: 5 warm-up steps (4 ms) left the first timed steps 8-10% slow
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--decode-iters", type=int, default=200)
    ap.add_argument("--quick", action="store_true", help="headline line only (no fp8 extras)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="",
                    help="profiling runs: comma list of prefill_bf16, prefill_fp8_block, prefill_fp8_mx, backward_fp8_mx, "
                         "decode_bf16, "
                         "decode_fp8_tensor, router, pages_shapes, copy (a plain 1 GiB device copy, the traffic-counter "
                         "reference); prints per-stage times instead of the JSON line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer's expert and tensor sharding over "
              "several GPUs is not built; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import routing_grouped_expert_index_amd as moe
    torch.cuda.set_device(0)
    if args.only:
        return profile_only(torch, moe, args)

    log("prefill bf16 T=8192 ...")
    pf = bench_prefill(torch, moe, "prefill_bf16", args.steps, args.warmup)
    wl = pf["wl"]
    ms = pf["dt"] / args.steps * 1e3
    value = wl.T * args.steps / pf["dt"]
    roof = roofline_gemm(wl, pf["gate_up_ms"], PEAK_BF16_TFLOPS)
    log(f"prefill bf16: {ms:.3f} ms/step, {value:.4g} tokens/s, gate_up {roof['achieved']} TFLOP/s")
    line = dict(metric=METRIC, value=round(value, 1), unit="tokens/s", n_gpus=1, steps=args.steps,
                warmup=args.warmup, ms_per_step=round(ms, 4), higher_is_better=True, scaling="weak",
                vs_baseline=None, dtype="bf16",
                data="synthetic: seeded N(0,1) bf16 activations, N(0,1)+Zipf-bias router logits, "
                     "N(0,0.02) bf16 expert weights",
                config=dict(workload="prefill_bf16", T=wl.T, H=wl.H, I=wl.I, E=wl.E, top_k=wl.k,
                            path=pf["path"], routing="softmax top-8 renormalised, Zipf-skewed load",
                            max_expert_rows=int(pf["counts"].max()), min_expert_rows=int(pf["counts"].min())),
                roofline=roof,
                layer=layer_fractions(wl, pf["dt"] / args.steps, PEAK_BF16_TFLOPS),
                stages_us={k: round(v * 1e3, 2) for k, v in pf["stages_ms"].items()})
    a, w = pf["host"]
    del pf["layer"]
    torch.cuda.empty_cache()

    log("decode bf16 B=1..4 (cold HBM) ...")
    line["decode"] = dict(workload="decode_bf16 H=2048 I=768 E=128 top-8", timing="cold HBM, median of "
                          f"{args.decode_iters}; us_per_layer: moe_route + moe_forward launched on "
                          "the stream between two HIP events (us_route, us_forward: the two calls "
                          "separately); us_forward_device: moe_forward's device span, first kernel start "
                          "to last kernel end, from events attached to those dispatches (moe_forward_timed), "
                          "hbm_frac_forward_device over it; us_per_layer_fused: moe_decode_forward, the "
                          "routing folded into "
                          "the route-direct Gate/Up kernel (one call); _graph: the same step replayed from "
                          "a HIP graph, cold; "
                          "_graph_warm: replayed back to back with the weights cached; dominant: "
                          "the kernel between stage events",
                          batches=bench_decode(torch, moe, "decode_bf16", (1, 2, 3, 4), args.decode_iters))
    torch.cuda.empty_cache()
    log("router scores + routing B=1..4 ...")
    line["router"] = dict(
        workload="router scores x W_r (fp32 [2048,128]) + top-8 routing, decode_bf16 shapes",
        timing=f"cold HBM, median of {args.decode_iters}, between two HIP events",
        batches=bench_router(torch, moe, (1, 2, 3, 4), args.decode_iters))
    torch.cuda.empty_cache()
    if not args.quick:
        log("dispatch crossover (cold, forced paths) ...")
        line["crossover"] = dict(
            timing="cold HBM, moe_route + moe_forward between two HIP events, median",
            decode_fp8_tensor=bench_crossover(torch, moe, "decode_fp8_tensor", range(1, 17), 30),
            decode_fp8_mx=bench_crossover(torch, moe, "decode_fp8_mx", range(1, 17), 30),
            decode_bf16=bench_crossover(torch, moe, "decode_bf16", range(1, 17), 30))
        torch.cuda.empty_cache()
        log("the pages' FP8 decode shapes, forward alone in a HIP graph ...")
        line["pages_shapes"] = dict(
            timing=f"moe_forward alone (routes given) captured in a HIP graph with preallocated output; "
                   f"cold: median of {args.decode_iters} replays after a 1 GiB read; warm: 200 back-to-back "
                   "replays; stream_cold: the same launches made straight on the stream, cold; stream_warm: "
                   "the same, without the read between calls (weights cache-resident), each call between its "
                   "own two events, median. pages_h20_us: "
                   "the forced route-direct single-op CUDA graph latency the pages print for the same shape "
                   "on an H20 (context)",
            shapes=bench_pages_shapes(torch, moe, args.decode_iters))
        torch.cuda.empty_cache()
        log("decode fp8 per-tensor B=1..4 ...")
        line["decode_fp8_per_tensor"] = dict(
            workload="decode_fp8_tensor H=4096 I=192 E=192 top-8",
            batches=bench_decode(torch, moe, "decode_fp8_tensor", (1, 2, 3, 4), args.decode_iters))
        torch.cuda.empty_cache()
        log("decode MX fp8 B=1..4 ...")
        line["decode_fp8_mx32"] = dict(
            workload="decode_fp8_mx H=4096 I=512 E=128 top-8, MX e4m3 (E8M0 per 32 along K)",
            batches=bench_decode(torch, moe, "decode_fp8_mx", (1, 2, 3, 4), args.decode_iters))
        torch.cuda.empty_cache()
        log("prefill fp8 block128 T=4096 ...")
        p5 = bench_prefill(torch, moe, "prefill_fp8_block", args.steps, args.warmup)
        w5 = p5["wl"]
        r5 = roofline_gemm(w5, p5["gate_up_ms"], PEAK_FP8_TFLOPS)
        line["prefill_fp8_block128"] = dict(
            workload="prefill_fp8_block T=4096 H=4096 I=512 E=128 top-8",
            tokens_per_s=round(w5.T * args.steps / p5["dt"], 1),
            ms_per_step=round(p5["dt"] / args.steps * 1e3, 4), roofline=r5,
            layer=layer_fractions(w5, p5["dt"] / args.steps, PEAK_FP8_TFLOPS),
            stages_us={k: round(v * 1e3, 2) for k, v in p5["stages_ms"].items()})
        del p5
        torch.cuda.empty_cache()
        log("prefill MX fp8 T=4096 ...")
        p6 = bench_prefill(torch, moe, "prefill_fp8_mx", args.steps, args.warmup)
        w6 = p6["wl"]
        line["prefill_fp8_mx32"] = dict(
            workload="prefill_fp8_mx T=4096 H=4096 I=512 E=128 top-8, MX e4m3 (E8M0 per 32 along K)",
            tokens_per_s=round(w6.T * args.steps / p6["dt"], 1),
            ms_per_step=round(p6["dt"] / args.steps * 1e3, 4),
            roofline=roofline_gemm(w6, p6["gate_up_ms"], PEAK_FP8_TFLOPS),
            layer=layer_fractions(w6, p6["dt"] / args.steps, PEAK_FP8_TFLOPS),
            stages_us={k: round(v * 1e3, 2) for k, v in p6["stages_ms"].items()})
        del p6
        torch.cuda.empty_cache()
        log("MX training backward T=4096 ...")
        line["backward_fp8_mx32"] = bench_backward(torch, moe, max(5, args.steps // 5), max(3, args.warmup // 10))
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline(a, w, wl)
    print(json.dumps(line), flush=True)
    recap(line)


# Time budgets of the targets (≥60% of HBM for the decode forward at B=1..4,
# ≥50% of dense MFMA for a prefill layer), from the bytes and flops each moves.
DECODE_BUDGET_US = {"decode": [15.7, 30.5, 44.3, 57.3], "decode_fp8_per_tensor": [3.94, 7.71, 11.32, 14.79]}
PREFILL_BUDGET_US = {"prefill_bf16": 494.8, "prefill_fp8_block128": 164.9, "prefill_fp8_mx32": 164.9}


def recap(line):
    """Compact stderr lines after the JSON line: every target next to its measurement."""
    for key, name in (("decode", "decode bf16 E128 H2048 I768"),
                      ("decode_fp8_per_tensor", "decode fp8 per-tensor E192 H4096 I192")):
        if key not in line:
            continue
        for B, r in line[key]["batches"].items():
            budget = DECODE_BUDGET_US[key][int(B) - 1]
            log(f"recap {name} B={B}: forward {r['us_forward']} us stream / {r['us_forward_device']} us device "
                f"(budget {budget}) = {r['hbm_frac_forward']:.3f} / {r['hbm_frac_forward_device']:.3f} of HBM over "
                f"{r['distinct_experts']} experts' weights; "
                f"route+forward {r['us_per_layer']} us; one call {r['us_per_layer_fused']} us; "
                f"{r['dominant']['kernel']} {r['dominant']['avg_launch_us']} us = {r['dominant']['frac']:.3f} of HBM")
    rows = [("prefill_bf16", line.get("layer"), line.get("roofline"), line.get("ms_per_step"), line.get("value"))]
    for key in ("prefill_fp8_block128", "prefill_fp8_mx32"):
        if key in line:
            rows.append((key, line[key]["layer"], line[key]["roofline"], line[key]["ms_per_step"],
                         line[key]["tokens_per_s"]))
    for key, lay, roof, ms, tps in rows:
        if lay is None:
            continue
        log(f"recap {key}: {ms * 1e3:.1f} us/layer (budget {PREFILL_BUDGET_US[key]}), {tps:.4g} tokens/s; layer "
            f"{lay['mfma_frac']:.3f} of MFMA, {lay['hbm_frac']:.3f} of HBM; Gate/Up {roof['avg_launch_us']} us = "
            f"{roof['frac']:.3f} of MFMA peak")
    bw = line.get("backward_fp8_mx32")
    if bw:
        dom = bw["dominant"]
        log(f"recap backward MX T=4096: {bw['ms_per_step'] * 1e3:.1f} us/step, {bw['tokens_per_s']:.4g} tokens/s; "
            f"dominant {dom['stage']} {dom['us']} us = {dom.get('frac', 0):.3f} of {dom.get('bound', '?')} peak; "
            f"training step (prepare + forward + backward) {bw['train_step_ms']:.3f} ms")
    cb = line.get("cpu_baseline")
    if cb:
        log(f"recap cpu oracle: {cb['value']} {cb['unit']} on {cb['cores']} threads ({cb['sample']})")


if __name__ == "__main__":
    main()
