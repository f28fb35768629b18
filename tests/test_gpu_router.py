"""GPU parity of the router scores and routing in one call (moe_route_project).

The scores x W_r are compared with the oracle's (fp64 sum, rounded once) within
the fp32 accumulation bound (H + 1) u sum_h |x_h w_he| + u |score|, u = 2^-24.
The top-k decision is an integer taken from floating point, so the routing is
compared bit for bit with the oracle's routing of the kernel's own fp32 scores.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, bf16_dev, check_routing, moe, oracle, random_activations, routes_np, say
from workloads import bf16_bits_to_f32

pytestmark = pytest.mark.gpu

U = 2.0 ** -24

CASES = [
    # (T, H, E, k)  -- one launch (scores + routing) unless noted
    (64, 256, 16, 8),      # the tiny layer: 8 token blocks x 4 K splits
    (1, 2048, 128, 8), (2, 2048, 128, 8), (3, 2048, 128, 8), (4, 2048, 128, 8),
    (5, 4096, 192, 8), (8, 4096, 192, 8), (16, 4096, 192, 8),
    (7, 128, 20, 3),       # E not a multiple of 64
    (3, 512, 512, 2),      # E = 512: two tokens per workgroup
    (2, 384, 512, 512),    # k = E = 512, six K splits
    (9, 64, 6, 6),         # one 64-row step, k = E
    (1, 64, 1, 1),
    (37, 320, 100, 7),     # ragged token blocks, five 64-row steps in one K split
    (512, 256, 16, 8),     # partials too large to stage: scores kernel, then the small routing kernel
    (3000, 512, 64, 4),    # scores kernel, then the three routing kernels
    (100, 2048, 512, 2),   # scores too large for one workgroup's LDS: scores kernel + small routing
    (4096, 128, 16, 1),
]


def _inputs(T, H, E, seed):
    a = random_activations(T, H, E, seed, logits="router")
    return a["x"], a["w_router"]


def _check_scores(g, x_bits, w):
    ref = oracle.router_logits(x_bits, w)
    mag = np.abs(bf16_bits_to_f32(x_bits).astype(np.float64)) @ np.abs(w.astype(np.float64))
    H = x_bits.shape[1]
    bound = (H + 1) * U * mag + U * np.abs(ref.astype(np.float64))
    err = np.abs(g.astype(np.float64) - ref.astype(np.float64))
    assert np.all(err <= bound), f"score error {err.max():.3e} over the bound"
    return ref


def _run(x_bits, w, k, **kw):
    r, lg = moe.route_project(bf16_dev(x_bits), torch.from_numpy(w).to(DEV), k, **kw)
    torch.cuda.synchronize()
    return r, lg


@pytest.mark.parametrize("T,H,E,k", CASES)
def test_route_project_parity(T, H, E, k):
    say(f"route_project T={T} H={H} E={E} k={k}")
    x_bits, w = _inputs(T, H, E, seed=T + H + E)
    r, lg = _run(x_bits, w, k)
    g = lg.cpu().numpy()
    _check_scores(g, x_bits, w)
    check_routing(routes_np(r), oracle.route(g, k))


def test_route_project_repeatable_with_shared_workspace():
    """Calls of several shapes on one workspace (its arrival counter must return to zero after
    each), every result checked, and a repeated call giving the same bits."""
    shapes = [(4, 2048, 128, 8), (64, 256, 16, 8), (1, 2048, 128, 8), (16, 4096, 192, 8), (4, 2048, 128, 8)]
    need = max(moe.route_project_workspace_size(*s) for s in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    first = {}
    for i, (T, H, E, k) in enumerate(shapes):
        x_bits, w = _inputs(T, H, E, seed=70 + T)
        r, lg = _run(x_bits, w, k, workspace=ws)
        g = lg.cpu().numpy()
        _check_scores(g, x_bits, w)
        check_routing(routes_np(r), oracle.route(g, k))
        if (T, H, E, k) in first:
            assert np.array_equal(first[(T, H, E, k)].view(np.int32), g.view(np.int32))
        first[(T, H, E, k)] = g
    assert int(ws[:4].view(torch.int32).item()) == 0


def test_route_project_empty_batch():
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((256, 16), dtype=torch.float32, device=DEV)
    r, lg = moe.route_project(x, w, 4)
    torch.cuda.synchronize()
    assert lg.shape == (0, 16)
    assert r.expert_counts.cpu().tolist() == [0] * 16
    assert r.expert_offsets.cpu().tolist() == [0] * 17
