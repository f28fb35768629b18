"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Routing (ids, counts, offsets, perm, route_pos) must match bit for bit and the
gates to 1e-6; outputs within max-abs 2e-2 and rel-L2 1e-2 (bf16) or rel-L2
2e-2 and cosine >= 0.999 (fp8), compared with the fp64 oracle.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import (DEV, WORKLOADS, bf16_dev, check_out, check_routing, moe, oracle, oracle_out,
                         random_activations, random_weights, routes_np, run, say, weights_dev,
                         workload_dev, workload_inputs, workload_weights)
from workloads import (_normal_per_expert, bf16_bits_to_f32, quantise_weight_block128, tie_heavy_logits,
                       to_bf16_bits)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ routing --
ROUTE_CASES = [
    # (T, E, k, kind)  -- small fused kernel and the three-kernel path, ragged sizes
    (64, 16, 8, "normal"), (1, 128, 8, "normal"), (4, 128, 8, "normal"), (8, 192, 8, "normal"),
    (8192, 128, 8, "zipf"), (4096, 128, 8, "normal"), (513, 64, 2, "normal"), (1000, 512, 20, "normal"),
    (3, 512, 512, "normal"), (5000, 7, 7, "normal"), (2000, 64, 8, "ties"), (300, 16, 8, "ties"),
    (0, 16, 4, "normal"), (1, 1, 1, "normal"), (777, 1, 1, "normal"), (65, 3, 2, "ties"),
]


@pytest.mark.parametrize("T,E,k,kind", ROUTE_CASES)
def test_route_parity(T, E, k, kind):
    say(f"route T={T} E={E} k={k} {kind}")
    if kind == "ties":
        lg = tie_heavy_logits(T, E, seed=T + E)
    else:
        lg = random_activations(T, 8, E, seed=1000 + T + E, logits="zipf" if kind == "zipf" else "normal")["logits"]
    r = moe.route(torch.from_numpy(lg).to(DEV), k)
    torch.cuda.synchronize()
    check_routing(routes_np(r), oracle.route(lg, k))


def test_route_equal_logits_all_experts():
    T, E = 50, 32
    lg = np.zeros((T, E), np.float32)
    r = routes_np(moe.route(torch.from_numpy(lg).to(DEV), E))
    assert np.array_equal(r["topk_ids"], np.tile(np.arange(E, dtype=np.int32), (T, 1)))
    assert np.all(r["topk_weights"] == np.float32(1.0 / E))
    check_routing(r, oracle.route(lg, E))


# -------------------------------------------------------------- forward ------
def _compare(name, x, lg, k, dev_w, host_w, quant, path, tokens=None):
    r, out = run(x, lg, k, dev_w, quant, path)
    ref_r = oracle.route(lg, k)
    check_routing(routes_np(r), ref_r)
    ref = oracle_out(x, ref_r, host_w, quant, tokens)
    got = out.float().cpu().numpy()
    if tokens is not None:
        got = got[tokens]
    return check_out(got, ref, "bf16" if quant == "bf16" else "fp8", f"{name} {path}")


@pytest.mark.parametrize("path", ["auto", "grouped", "route_direct"])
def test_tiny_bf16(path):
    """The tiny layer end to end: router scores and routing in one call, then the layer; the
    oracle routes the kernel's fp32 scores (checked against its own) and computes the layer."""
    name = "tiny_bf16"
    wl = WORKLOADS[name]
    a = workload_inputs(name)
    pw, _ = workload_dev(name)
    r, lg = moe.route_project(bf16_dev(a["x"]), torch.from_numpy(a["w_router"]).to(DEV), wl.k)
    out = moe.forward(bf16_dev(a["x"]), r, pw, path=path)
    torch.cuda.synchronize()
    g = lg.cpu().numpy()
    ref_lg = oracle.router_logits(a["x"], a["w_router"])
    assert np.max(np.abs(g - ref_lg)) <= 1e-5
    ref_r = oracle.route(g, wl.k)
    check_routing(routes_np(r), ref_r)
    # the kernel's scores pick the same routes as the oracle's own scores (no near-tie flips)
    check_routing(ref_r, oracle.route(ref_lg, wl.k))
    ref = oracle_out(a["x"], ref_r, workload_weights(name), "bf16")
    check_out(out.float().cpu().numpy(), ref, "bf16", f"{name} {path}")


@pytest.mark.parametrize("path", ["auto", "grouped", "route_direct"])
def test_tiny_bf16_host_logits(path):
    """The tiny layer with its router scores computed by the oracle on the host and fed to
    moe_route: every value the reference uses comes from the host, none from the GPU."""
    name = "tiny_bf16"
    wl = WORKLOADS[name]
    a = workload_inputs(name)
    lg = oracle.router_logits(a["x"], a["w_router"])
    _compare(f"{name} host logits", a["x"], lg, wl.k, workload_dev(name), workload_weights(name), "bf16", path)


@pytest.mark.parametrize("B", [1, 2, 3, 4])
@pytest.mark.parametrize("path", ["auto", "grouped"])
def test_decode_bf16(B, path):
    name = "decode_bf16"
    a = workload_inputs(name, batch=B)
    _compare(f"{name} B={B}", a["x"], a["logits"], 8, workload_dev(name), workload_weights(name), "bf16", path)


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("path", ["auto", "grouped", "route_direct"])
def test_decode_fp8_per_tensor(B, path):
    name = "decode_fp8_tensor"
    a = workload_inputs(name, batch=B)
    _compare(f"{name} B={B}", a["x"], a["logits"], 8, workload_dev(name), workload_weights(name),
             "fp8_per_tensor", path)


def _sample_tokens(T, n, seed):
    rng = np.random.default_rng(seed)
    t = np.unique(np.concatenate([[0, 1, T - 1], rng.choice(T, n, replace=False)]))
    return t.astype(np.int32)


@pytest.mark.parametrize("name", ["prefill_bf16", "prefill_fp8_block"])
def test_prefill_whole_output(name):
    """Full-size prefill (the benchmarked launch, every row tile of both grouped GEMMs): the
    whole [T, H] output against the oracle's, routing bit-exact."""
    wl = WORKLOADS[name]
    a = workload_inputs(name)
    say(f"{name}: whole output, T={wl.T}")
    _compare(name, a["x"], a["logits"], wl.k, workload_dev(name), workload_weights(name), wl.quant, "auto")


@pytest.mark.parametrize("quant", ["bf16", "fp8_block128"])
def test_large_t_intermediates_past_2gib(quant):
    """T=70000, k=E=8: the sorted Down output y is 70000*8*2048*2 = 2.3 GB (past the 2^31
    byte offsets of a single buffer resource), so its row tiles are addressed from 64-bit
    bases; compared on the first and last tokens (the highest y rows of every expert) and a
    random sample, routing bit-exact."""
    T, H, I, E, k = 70000, 2048, 256, 8, 8
    say(f"large T={T} H={H} I={I} E={E} k={k} {quant}")
    a = random_activations(T, H, E, seed=77)
    w = random_weights(E, H, I, quant, seed=78)
    assert moe.select_path(T, H, I, E, k, quant) == "grouped"
    tok = np.unique(np.concatenate([np.arange(4), np.arange(T - 40, T), _sample_tokens(T, 40, 79)])).astype(np.int32)
    _compare(f"large T {quant}", a["x"], a["logits"], k, weights_dev(w, quant), w, quant, "grouped", tok)


# -------------------------------------------------------------- edge cases --
EDGE = [
    # (T, H, I, E, k, quant, logits, tag)
    (37, 256, 128, 8, 2, "bf16", "normal", "ragged tiles"),
    (300, 256, 128, 4, 1, "bf16", "normal", "multi-tile experts"),
    (5, 256, 64, 1, 1, "bf16", "normal", "E=1"),
    (9, 128, 64, 6, 6, "bf16", "normal", "k=E"),
    (1, 256, 128, 64, 8, "bf16", "normal", "T=1 most experts empty"),
    (200, 256, 128, 16, 4, "bf16", "hot", "all routes to few experts"),
    (20, 256, 192, 12, 3, "fp8_per_tensor", "normal", "per-tensor I%128!=0"),
    (150, 384, 256, 8, 2, "fp8_per_tensor", "normal", "per-tensor multi-tile"),
    (70, 256, 256, 6, 2, "fp8_block128", "normal", "block128 ragged"),
    (3, 512, 128, 32, 4, "fp8_block128", "normal", "block128 decode"),
    # route-direct Gate/Up row split with per-lane 128-block scales (split 2, then 4)
    (1, 4096, 512, 128, 8, "fp8_block128", "normal", "block128 B=1 row split 2"),
    (1, 8192, 128, 8, 2, "fp8_block128", "normal", "block128 row split 4"),
    # grids of fewer than 8 workgroups with several n-tiles (every tile range must be walked)
    (5, 256, 192, 1, 1, "bf16", "normal", "small grid, 3 n-tiles"),
    (3, 256, 384, 1, 1, "fp8_block128", "normal", "small grid block128"),
    (2, 384, 192, 1, 1, "fp8_per_tensor", "normal", "small grid per-tensor"),
    # H a multiple of 64 but not of 128 (the Down GEMM's last 512-column tile mostly past H)
    (13, 192, 128, 8, 2, "bf16", "normal", "H=192"),
    (150, 192, 256, 8, 2, "bf16", "normal", "H=192 multi-tile"),
    (7, 320, 192, 6, 3, "fp8_per_tensor", "normal", "H=320 per-tensor"),
    (90, 576, 128, 10, 4, "fp8_per_tensor", "normal", "H=576 per-tensor multi-tile"),
]


# route-direct Gate/Up row split each row-split case exists to exercise
EXPECT_SPLIT = {"block128 B=1 row split 2": 2, "block128 row split 4": 4}


@pytest.mark.parametrize("T,H,I,E,k,quant,kind,tag", EDGE)
@pytest.mark.parametrize("path", ["grouped", "route_direct"])
def test_edge_cases(T, H, I, E, k, quant, kind, tag, path):
    say(f"edge {tag}: T={T} H={H} I={I} E={E} k={k} {quant} {path}")
    if path == "route_direct" and tag in EXPECT_SPLIT:
        li = moe.forward_launch_info(T, H, I, E, k, quant, path)
        say(f"  launch {li}")
        assert li["gate_up_split"] == EXPECT_SPLIT[tag], li
    a = random_activations(T, H, E, seed=T * 7 + E)
    lg = a["logits"]
    if kind == "hot":
        lg = lg.copy()
        lg[:, :k] += 50.0       # every token picks experts 0..k-1
    w = random_weights(E, H, I, quant, seed=E * 13 + I)
    _compare(tag, a["x"], lg, k, weights_dev(w, quant), w, quant, path)


def test_empty_batch():
    w = random_weights(4, 128, 64, "bf16", seed=3)
    pw, _ = weights_dev(w, "bf16")
    r = moe.route(torch.zeros((0, 4), dtype=torch.float32, device=DEV), 2)
    out = moe.forward(torch.zeros((0, 128), dtype=torch.bfloat16, device=DEV), r, pw)
    torch.cuda.synchronize()
    assert out.shape == (0, 128)
    assert r.expert_counts.cpu().tolist() == [0] * 4
    assert r.expert_offsets.cpu().tolist() == [0] * 5


# ------------------------------------------------------------- determinism --
@pytest.mark.parametrize("name,path", [("prefill_bf16", "auto"), ("decode_fp8_tensor", "auto"),
                                       ("decode_bf16", "grouped"), ("prefill_fp8_block", "auto")])
def test_two_runs_bitwise_equal(name, path):
    wl = WORKLOADS[name]
    a = workload_inputs(name, batch=4 if wl.batches else None)
    _, o1 = run(a["x"], a["logits"], wl.k, workload_dev(name), wl.quant, path)
    _, o2 = run(a["x"], a["logits"], wl.k, workload_dev(name), wl.quant, path)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("name", ["decode_bf16", "decode_fp8_tensor", "decode_fp8_mx", "tiny_bf16"])
def test_graph_replay_bitwise_equal(name):
    wl = WORKLOADS[name]
    a = workload_inputs(name, batch=4 if wl.batches else None)
    pw, scales = workload_dev(name)
    x = bf16_dev(a["x"])
    T = x.shape[0]
    routes = moe.Routes(T, wl.E, wl.k, DEV)
    out = torch.empty((T, wl.H), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(256, moe.forward_workspace_size(T, wl.H, wl.I, wl.E, wl.k, wl.quant)),
                     dtype=torch.uint8, device=DEV)
    if "w_router" in a:   # router scores and routing in one launch (arrival counter in rws)
        wr = torch.from_numpy(a["w_router"]).to(DEV)
        lg = torch.empty((T, wl.E), dtype=torch.float32, device=DEV)
        rws = torch.zeros(moe.route_project_workspace_size(T, wl.H, wl.E, wl.k), dtype=torch.uint8, device=DEV)

        def route_step():
            moe.route_project(x, wr, wl.k, out=routes, logits=lg, workspace=rws)
    else:
        lg = torch.from_numpy(a["logits"]).to(DEV)
        rws_n = moe.route_workspace_size(T, wl.E, wl.k)
        rws = torch.empty(max(rws_n, 256), dtype=torch.uint8, device=DEV) if rws_n else None

        def route_step():
            moe.route(lg, wl.k, out=routes, workspace=rws)

    def step():
        route_step()
        moe.forward(x, routes, pw, quant=wl.quant, scales=scales, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
        step()      # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("path", ["grouped", "route_direct"])
def test_block128_wide_scale_range(path):
    """Blockwise FP8 with 128-channel K blocks whose magnitudes differ by up to 1e4 (activations
    1e-2..1e2, weights 0.1..10 per K block): the blockwise GEMMs keep their accumulators in the
    current K block's scale units, so consecutive blocks' scale ratios are far from 1.  Gate/Up
    has 8 K blocks, Down 3, and the second Gate/Up column tile has waves past N."""
    T, H, I, E, k = 37, 1024, 384, 6, 2
    say(f"block128 wide scale range T={T} H={H} I={I} E={E} k={k} {path}")
    a = random_activations(T, H, E, seed=91)
    fx = np.array([1e-2, 1.0, 1e2, 1e-1, 10.0, 1.0, 3e-2, 30.0], np.float32)
    x_bits = to_bf16_bits(bf16_bits_to_f32(a["x"]) * np.repeat(fx, 128)[None, :])
    gw = np.array([0.1, 10.0, 1.0, 0.3, 3.0, 1.0, 10.0, 0.1], np.float32)
    wgu = _normal_per_expert((E, H, 2 * I), 17, 0, 0.02) * np.repeat(gw, 128)[None, :, None]
    wd = _normal_per_expert((E, I, H), 17, 1, 0.02) * np.repeat(gw[:3], 128)[None, :, None]
    qgu, sgu = quantise_weight_block128(wgu)
    qd, sd = quantise_weight_block128(wd)
    w = dict(w_gate_up=qgu, w_down=qd, s_gate_up=sgu, s_down=sd)
    _compare("block128 wide scale range", x_bits, a["logits"], k, weights_dev(w, "fp8_block128"), w,
             "fp8_block128", path)


@pytest.mark.parametrize("name,B,path", [("decode_fp8_tensor", 2, "route_direct"), ("decode_bf16", 3, "grouped")])
def test_forward_timed_same_bits(name, B, path):
    """moe_forward_timed runs moe_forward's launches with events attached to the first and last
    dispatch: the same output bits, and a positive device span."""
    wl = WORKLOADS[name]
    a = workload_inputs(name, batch=B)
    pw, sc = workload_dev(name)
    x = bf16_dev(a["x"])
    r = moe.route(torch.from_numpy(a["logits"]).to(DEV), wl.k)
    ref = moe.forward(x, r, pw, scales=sc, path=path)
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = moe.forward(x, r, pw, scales=sc, path=path, device_events=(d0, d1))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    span = d0.elapsed_time(d1)
    say(f"  {name} B={B} {path}: device span {span * 1e3:.2f} us")
    assert 0.0 < span < 10.0


@pytest.mark.parametrize("name,B,path", [("decode_fp8_tensor", 2, "route_direct"), ("decode_bf16", 3, "grouped"),
                                         ("prefill_fp8_block", None, "grouped")])
def test_forward_profiled_stage_events(name, B, path):
    """moe_forward_profiled attaches its events to the kernel dispatches: the same output bits as
    moe_forward, every stage a positive device time, and the stages adding up to the span from
    the first kernel's start to the last kernel's end (events[-1] - events[0])."""
    wl = WORKLOADS[name]
    a = workload_inputs(name, batch=B)
    pw, sc = workload_dev(name)
    x = bf16_dev(a["x"])
    r = moe.route(torch.from_numpy(a["logits"]).to(DEV), wl.k)
    ref = moe.forward(x, r, pw, scales=sc, path=path)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    out, names = moe.forward(x, r, pw, scales=sc, path=path, events=evs)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    n = len(names)
    stages = [evs[i].elapsed_time(evs[i + 1]) for i in range(n)]
    total = evs[0].elapsed_time(evs[n])
    say(f"  {name} {path}: {dict(zip(names, [round(s * 1e3, 2) for s in stages]))} us, span {total * 1e3:.2f} us")
    assert all(s > 0.0 for s in stages)
    assert abs(sum(stages) - total) <= 1e-3 * total + 1e-6
