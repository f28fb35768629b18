"""moe_decode_forward: the routing folded into the route-direct Gate/Up kernel.  The output and
the written routes must equal, bit for bit, moe_route followed by moe_forward on the same inputs
(the same top-k code and the same kernels after it), and the layer the oracle's."""
import numpy as np
import pytest
import torch

from gpu_helpers import (DEV, WORKLOADS, bf16_dev, check_out, check_routing, moe, oracle, oracle_out,
                         random_activations, random_weights, routes_np, say, weights_dev, workload_dev,
                         workload_inputs, workload_weights)
from workloads import tie_heavy_logits

pytestmark = pytest.mark.gpu


def _both(x_bits, lg, k, dev_w, quant, **kw):
    pw, sc = dev_w
    x = bf16_dev(x_bits)
    lgd = torch.from_numpy(np.ascontiguousarray(lg)).to(DEV)
    r = moe.route(lgd, k)
    ref = moe.forward(x, r, pw, quant=quant, scales=sc, path="route_direct", **kw)
    out, rf = moe.decode_forward(lgd, x, k, pw, quant=quant, scales=sc, path="route_direct", **kw)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "fused output differs from route + forward"
    assert torch.equal(rf.topk_ids, r.topk_ids)
    assert torch.equal(rf.topk_weights.view(torch.int32), r.topk_weights.view(torch.int32))
    return out, r


@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_decode_fused_bf16(B):
    name = "decode_bf16"
    a = workload_inputs(name, batch=B)
    out, r = _both(a["x"], a["logits"], 8, workload_dev(name), "bf16")
    ref_r = oracle.route(a["logits"], 8)
    check_routing({**routes_np(r)}, ref_r)
    check_out(out.float().cpu().numpy(), oracle_out(a["x"], ref_r, workload_weights(name), "bf16"), "bf16",
              f"fused decode bf16 B={B}")


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 6, 7, 8])
def test_decode_fused_fp8_per_tensor(B):
    name = "decode_fp8_tensor"
    a = workload_inputs(name, batch=B)
    out, _ = _both(a["x"], a["logits"], 8, workload_dev(name), "fp8_per_tensor")
    if B in (1, 8):
        ref_r = oracle.route(a["logits"], 8)
        check_out(out.float().cpu().numpy(), oracle_out(a["x"], ref_r, workload_weights(name), "fp8_per_tensor"),
                  "fp8", f"fused decode fp8 B={B}")


EDGE = [
    # (T, H, I, E, k, quant, kind)
    (3, 512, 256, 32, 4, "fp8_block128", "normal"),
    (2, 256, 128, 20, 3, "bf16", "normal"),        # E not a multiple of 64
    (3, 256, 128, 512, 2, "bf16", "normal"),       # E = 512
    (4, 256, 128, 8, 8, "fp8_per_tensor", "normal"),   # k = E
    (5, 256, 128, 16, 4, "bf16", "ties"),          # exact ties go to the lower id
]


@pytest.mark.parametrize("T,H,I,E,k,quant,kind", EDGE)
def test_decode_fused_edge(T, H, I, E, k, quant, kind):
    say(f"fused decode edge T={T} H={H} I={I} E={E} k={k} {quant} {kind}")
    a = random_activations(T, H, E, seed=500 + E)
    lg = tie_heavy_logits(T, E, seed=501) if kind == "ties" else a["logits"]
    w = random_weights(E, H, I, quant, seed=502 + E)
    out, r = _both(a["x"], lg, k, weights_dev(w, quant), quant)
    ref_r = oracle.route(lg, k)
    assert np.array_equal(r.topk_ids.cpu().numpy(), ref_r["topk_ids"])
    check_out(out.float().cpu().numpy(), oracle_out(a["x"], ref_r, w, quant), "bf16" if quant == "bf16" else "fp8",
              f"fused edge {quant}")


def test_decode_fused_expert_slice_accumulate():
    T, H, I, E, k = 3, 256, 128, 16, 4
    a = random_activations(T, H, E, seed=510)
    w = random_weights(E, H, I, "bf16", seed=511)
    e0, n = 5, 7
    ws = {key: (None if w[key] is None else np.ascontiguousarray(w[key][e0:e0 + n])) for key in w}
    start = torch.randn((T, H), device=DEV).to(torch.bfloat16)
    o1 = start.clone()
    o2 = start.clone()
    pw, _ = weights_dev(ws, "bf16")
    lgd = torch.from_numpy(a["logits"]).to(DEV)
    r = moe.route(lgd, k)
    moe.forward(bf16_dev(a["x"]), r, pw, out=o1, path="route_direct", expert_begin=e0, num_experts=n,
                accumulate=True)
    moe.decode_forward(lgd, bf16_dev(a["x"]), k, pw, out=o2, path="route_direct", expert_begin=e0,
                       num_experts=n, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_decode_fused_rejects_grouped_and_empty_batch():
    w = random_weights(4, 128, 64, "bf16", seed=520)
    pw, _ = weights_dev(w, "bf16")
    x = torch.zeros((40, 128), dtype=torch.bfloat16, device=DEV)
    lg = torch.zeros((40, 4), dtype=torch.float32, device=DEV)
    with pytest.raises(moe.MoeError):
        moe.decode_forward(lg, x, 2, pw)               # AUTO picks grouped for 80 routes over 4 experts
    out, r = moe.decode_forward(torch.zeros((0, 4), device=DEV), torch.zeros((0, 128), dtype=torch.bfloat16,
                                device=DEV), 2, pw, path="route_direct")
    torch.cuda.synchronize()
    assert out.shape == (0, 128)


def test_decode_fused_graph_replay():
    """Captured in a HIP graph and replayed several times with eager calls between: every replay
    gives the eager output's bits and the same routes."""
    name = "decode_fp8_tensor"
    wl = WORKLOADS[name]
    a = workload_inputs(name, batch=3)
    pw, sc = workload_dev(name)
    x = bf16_dev(a["x"])
    lg = torch.from_numpy(a["logits"]).to(DEV)
    T = x.shape[0]
    routes = moe.Routes(T, wl.E, wl.k, DEV)
    out = torch.empty((T, wl.H), dtype=torch.bfloat16, device=DEV)
    ws = torch.zeros(max(256, moe.forward_workspace_size(T, wl.H, wl.I, wl.E, wl.k, wl.quant)), dtype=torch.uint8,
                     device=DEV)

    def step():
        moe.decode_forward(lg, x, wl.k, pw, quant=wl.quant, scales=sc, out=out, routes=routes, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager, ids = out.clone(), routes.topk_ids.clone()
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
        routes.topk_ids.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
        assert torch.equal(routes.topk_ids, ids)
        step()
        torch.cuda.synchronize()
