"""GPU parity of expert-parallel slices and the shared output (moe_forward_ex).

One call holds the weights of experts [e0, e0 + n) only, the routes stay global,
and routes to other experts add nothing ("perf: add small-batch route MMA for
MoE", Summary: the fast path keeps EP routing and the shared output).  Each
slice is compared with the oracle's slice forward on the same sliced weights;
tokens without a route into the slice must come out exactly zero; accumulating
slices into one output must match the sum of the slices.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, bf16_dev, check_out, moe, oracle, random_activations, random_weights, say, \
    weights_dev
from workloads import bf16_bits_to_f32, to_bf16_bits

pytestmark = pytest.mark.gpu

SLICES = ((0, 5), (5, 8), (13, 3))      # a partition of E = 16 into unequal slices
KIND = {"bf16": "bf16", "fp8_per_tensor": "fp8", "fp8_block128": "fp8"}


def _slice_w(w, e0, n):
    out = dict(w_gate_up=np.ascontiguousarray(w["w_gate_up"][e0:e0 + n]),
               w_down=np.ascontiguousarray(w["w_down"][e0:e0 + n]))
    for key in ("s_gate_up", "s_down"):
        out[key] = None if w[key] is None else np.ascontiguousarray(w[key][e0:e0 + n])
    return out


def _oracle_slice(x_bits, r, w_s, quant, e0):
    return oracle.forward(x_bits, r["topk_ids"], r["topk_weights"], w_s["w_gate_up"], w_s["w_down"],
                          quant=quant, s_gate_up=w_s["s_gate_up"], s_down=w_s["s_down"], expert_begin=e0)


def _routes(lg, k):
    r = moe.route(torch.from_numpy(np.ascontiguousarray(lg)).to(DEV), k)
    torch.cuda.synchronize()
    return r, oracle.route(lg, k)


@pytest.mark.parametrize("T,H,I", [(6, 512, 256), (150, 256, 128)])
@pytest.mark.parametrize("quant", ["bf16", "fp8_per_tensor", "fp8_block128"])
@pytest.mark.parametrize("path", ["grouped", "route_direct"])
def test_ep_slices_and_shared_output(T, H, I, quant, path):
    E, k = 16, 4
    say(f"ep slices T={T} H={H} I={I} E={E} k={k} {quant} {path}")
    a = random_activations(T, H, E, seed=300 + T)
    w = random_weights(E, H, I, quant, seed=301 + I)
    r, ref_r = _routes(a["logits"], k)
    x = bf16_dev(a["x"])
    shared = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    total = np.zeros((T, H))
    for e0, n in SLICES:
        w_s = _slice_w(w, e0, n)
        pw, sc = weights_dev(w_s, quant)
        got = moe.forward(x, r, pw, quant=quant, scales=sc, path=path, expert_begin=e0, num_experts=n)
        moe.forward(x, r, pw, quant=quant, scales=sc, out=shared, path=path, expert_begin=e0,
                    num_experts=n, accumulate=True)
        torch.cuda.synchronize()
        ref = _oracle_slice(a["x"], ref_r, w_s, quant, e0)
        g = got.float().cpu().numpy()
        check_out(g, ref, KIND[quant], f"slice [{e0},{e0 + n})")
        ids = ref_r["topk_ids"]
        none_local = ~np.any((ids >= e0) & (ids < e0 + n), axis=1)
        assert np.all(g[none_local] == 0.0), "a token without routes into the slice is not zero"
        total += ref
    check_out(shared.float().cpu().numpy(), total, KIND[quant], "slices accumulated")


@pytest.mark.parametrize("path", ["grouped", "route_direct"])
def test_ep_full_slice_equals_layer(path):
    """The slice of all experts without accumulation is the plain layer, bit for bit."""
    T, H, I, E, k = 5, 512, 256, 16, 4
    a = random_activations(T, H, E, seed=310)
    w = random_weights(E, H, I, "fp8_per_tensor", seed=311)
    pw, sc = weights_dev(w, "fp8_per_tensor")
    r, _ = _routes(a["logits"], k)
    x = bf16_dev(a["x"])
    o1 = moe.forward(x, r, pw, quant="fp8_per_tensor", scales=sc, path=path)
    o2 = moe.forward(x, r, pw, quant="fp8_per_tensor", scales=sc, path=path, expert_begin=0,
                     num_experts=E)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("path", ["grouped", "route_direct"])
def test_ep_accumulate_onto_existing_output(path):
    """out = bf16(out + slice sum): one rounding of the fp32 sum, checked against the fp64 oracle
    plus the starting output."""
    T, H, I, E, k = 7, 256, 128, 16, 4
    e0, n = 4, 6
    a = random_activations(T, H, E, seed=320)
    w = random_weights(E, H, I, "bf16", seed=321)
    w_s = _slice_w(w, e0, n)
    pw, _ = weights_dev(w_s, "bf16")
    r, ref_r = _routes(a["logits"], k)
    rng = np.random.default_rng(322)
    start = to_bf16_bits(rng.normal(0.0, 0.05, (T, H)).astype(np.float32))
    out = bf16_dev(start)
    moe.forward(bf16_dev(a["x"]), r, pw, out=out, path=path, expert_begin=e0, num_experts=n,
                accumulate=True)
    torch.cuda.synchronize()
    ref = bf16_bits_to_f32(start).astype(np.float64) + _oracle_slice(a["x"], ref_r, w_s, "bf16", e0)
    check_out(out.float().cpu().numpy(), ref, "bf16", "accumulate")


@pytest.mark.parametrize("quant", ["bf16", "fp8_per_tensor"])
@pytest.mark.parametrize("path", ["grouped", "route_direct"])
def test_ep_slice_without_routes(quant, path):
    """Every token routes to experts 0..k-1; the slice [E-3, E) receives nothing: its output is
    exactly zero, and accumulating it leaves the shared output's bits unchanged."""
    T, H, I, E, k = 6, 256, 128, 16, 4
    e0, n = 13, 3
    a = random_activations(T, H, E, seed=330)
    lg = a["logits"].copy()
    lg[:, :k] += 50.0
    w = random_weights(E, H, I, quant, seed=331)
    pw, sc = weights_dev(_slice_w(w, e0, n), quant)
    r, ref_r = _routes(lg, k)
    assert not np.any(ref_r["topk_ids"] >= e0)
    x = bf16_dev(a["x"])
    got = moe.forward(x, r, pw, quant=quant, scales=sc, path=path, expert_begin=e0, num_experts=n)
    rng = np.random.default_rng(332)
    start = to_bf16_bits(rng.uniform(0.5, 1.0, (T, H)).astype(np.float32))   # no -0.0
    out = bf16_dev(start)
    moe.forward(x, r, pw, quant=quant, scales=sc, out=out, path=path, expert_begin=e0, num_experts=n,
                accumulate=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(got.float()).item() == 0
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), start)
