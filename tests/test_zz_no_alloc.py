"""moe_decode_forward_noalloc, the decode entry for callers that cannot allocate, through
the C ABI: the same kernels as moe_decode_forward with the workspace in the library's own
static device array, so the output and the written routes must equal moe_decode_forward's
(caller workspace) bit for bit -- on two calls in a row, the second with a smaller batch
(the array keeps the first call's contents)."""
import numpy as np
import pytest
import torch

from gpu_helpers import (DEV, WORKLOADS, bf16_dev, check_out, moe, oracle, oracle_out, random_activations,
                         random_weights, say, weights_dev, workload_dev, workload_inputs, workload_weights)

pytestmark = pytest.mark.gpu


def _pair(lg_np, x_bits, k, pw, sc, E, H):
    B = x_bits.shape[0]
    lg = torch.from_numpy(np.ascontiguousarray(lg_np)).to(DEV)
    x = bf16_dev(x_bits)
    ref, r_ref = moe.decode_forward(lg, x, k, pw, scales=sc)
    out = torch.full((B, H), float("nan"), dtype=torch.bfloat16, device=DEV)
    routes = moe.Routes(B, E, k, DEV)
    moe.decode_forward_noalloc(lg, x, k, pw, out, routes, scales=sc)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "output differs from moe_decode_forward"
    assert torch.equal(routes.topk_ids, r_ref.topk_ids)
    assert torch.equal(routes.topk_weights.view(torch.int32), r_ref.topk_weights.view(torch.int32))
    return out


@pytest.mark.parametrize("name,batches", [("decode_bf16", (4, 2)), ("decode_fp8_tensor", (8, 3)),
                                          ("decode_fp8_mx", (3, 1))])
def test_noalloc_matches_decode_forward(name, batches):
    wl = WORKLOADS[name]
    pw, sc = workload_dev(name)
    for B in batches:
        say(f"noalloc {name} B={B}")
        a = workload_inputs(name, batch=B)
        out = _pair(a["logits"], a["x"], wl.k, pw, sc, wl.E, wl.H)
        ref = oracle_out(a["x"], oracle.route(a["logits"], wl.k), workload_weights(name), wl.quant)
        check_out(out.float().cpu().numpy(), ref, "bf16" if wl.quant == "bf16" else "fp8", f"noalloc {name} B={B}")


def test_noalloc_blockwise_two_calls():
    E, H, I, k = 32, 2048, 768, 8
    w = random_weights(E, H, I, "fp8_block128", seed=90)
    pw, sc = weights_dev(w, "fp8_block128")
    for B in (3, 1):
        say(f"noalloc block128 E={E} H={H} I={I} B={B}")
        a = random_activations(B, H, E, seed=91 + B)
        _pair(a["logits"], a["x"], k, pw, sc, E, H)


def test_noalloc_rejects_oversize_before_launch():
    """A shape whose route-direct workspace exceeds the 16 MiB array is refused on the host."""
    T, H, I, E, k = 64, 8192, 2048, 512, 8
    assert moe.forward_workspace_size(T, H, I, E, k, "fp8_block128", "route_direct") > 16 << 20
    w = random_weights(2, 256, 128, "fp8_block128", seed=92)   # any packed weights: rejected first
    pw, sc = weights_dev(w, "fp8_block128")
    lg = torch.zeros((T, E), dtype=torch.float32, device=DEV)
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoeError) as ei:
        moe.decode_forward_noalloc(lg, x, k, pw, out, moe.Routes(T, E, k, DEV), scales=sc, path="route_direct")
    assert ei.value.code == -2 and "static scratch" in str(ei.value)
