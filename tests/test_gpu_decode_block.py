"""Route-direct blockwise FP8 decode at the two blockwise shapes the benchmark times
(E=128 with H=2048, I=768 and with H=4096, I=512; top-8; B=1..8; the benchmark's own
weights and activations): moe_forward on the forced route-direct path and on AUTO, and the
decode entry with the routing folded in (bit-identical to moe_route + moe_forward), against
the oracle ("perf: add small-batch route MMA for MoE", Performance: the blockwise tables).
Each case prints the launch shape it ran."""
import functools

import numpy as np
import pytest
import torch

from gpu_helpers import (DEV, bf16_dev, check_out, check_routing, moe, oracle, oracle_out, random_activations,
                         random_weights, routes_np, say, weights_dev, workload_weights)

pytestmark = pytest.mark.gpu

SHAPES = {
    "E128_H2048_I768": (128, 2048, 768, lambda: random_weights(128, 2048, 768, "fp8_block128", 6)),
    "E128_H4096_I512": (128, 4096, 512, lambda: workload_weights("prefill_fp8_block")),
}


@functools.lru_cache(maxsize=1)
def _weights(shape):
    w = SHAPES[shape][3]()
    return w, weights_dev(w, "fp8_block128")


@pytest.mark.parametrize("shape,B", [(s, B) for s in SHAPES for B in range(1, 9)])
def test_block128_decode_shapes(shape, B):
    E, H, I, _ = SHAPES[shape]
    k = 8
    w, (pw, sc) = _weights(shape)
    a = random_activations(B, H, E, 20000 + B)      # the benchmark's activations for this B
    li = moe.forward_launch_info(B, H, I, E, k, "fp8_block128", "route_direct")
    say(f"block128 decode {shape} B={B}: launch {li}")
    x = bf16_dev(a["x"])
    lgd = torch.from_numpy(a["logits"]).to(DEV)
    r = moe.route(lgd, k)
    out_rd = moe.forward(x, r, pw, scales=sc, path="route_direct")
    out_auto = moe.forward(x, r, pw, scales=sc, path="auto")
    out_fused, rf = moe.decode_forward(lgd, x, k, pw, scales=sc, path="route_direct")
    torch.cuda.synchronize()
    assert torch.equal(out_fused.view(torch.int16), out_rd.view(torch.int16)), "fused decode differs"
    assert torch.equal(rf.topk_ids, r.topk_ids)
    ref_r = oracle.route(a["logits"], k)
    check_routing(routes_np(r), ref_r)
    ref = oracle_out(a["x"], ref_r, w, "fp8_block128")
    check_out(out_rd.float().cpu().numpy(), ref, "fp8", f"{shape} B={B} route_direct")
    check_out(out_auto.float().cpu().numpy(), ref, "fp8", f"{shape} B={B} auto")
