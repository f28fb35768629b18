"""GPU parity of MX FP8 (e4m3 with an E8M0 power-of-two scale per 32 values along K) on the
grouped and route-direct paths, against the oracle's MX forward ("[mxfp8 moe training] add per
group blocked scale kernels", Summary: mxfp8 scales); tolerance as for the other FP8 modes."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, bf16_dev, check_out, check_routing, moe, oracle, oracle_out, random_activations, \
    random_weights, routes_np, say, weights_dev
from workloads import _normal_per_expert, bf16_bits_to_f32, quantise_weight_mx32, to_bf16_bits

pytestmark = pytest.mark.gpu


def _layer(x_bits, lg, k, w, tokens=None, **kw):
    pw, sc = weights_dev(w, "fp8_mx32")
    r = moe.route(torch.from_numpy(np.ascontiguousarray(lg)).to(DEV), k)
    out = moe.forward(bf16_dev(x_bits), r, pw, quant="fp8_mx32", scales=sc, **kw)
    torch.cuda.synchronize()
    ref_r = oracle.route(lg, k)
    check_routing(routes_np(r), ref_r)
    ref = oracle_out(x_bits, ref_r, w, "fp8_mx32", tokens)
    got = out.float().cpu().numpy()
    return (got if tokens is None else got[tokens]), ref


MX_CASES = [
    # (T, H, I, E, k, tag)
    (37, 256, 256, 6, 2, "ragged tiles"),
    (300, 512, 256, 8, 2, "multi-tile experts"),
    (5, 256, 512, 1, 1, "E=1, small grid, 2 n-tiles"),
    (64, 256, 512, 16, 8, "tiny layer shape"),
    (3, 1024, 768, 32, 4, "decode-sized, K groups of Down 3"),
    (200, 2048, 768, 16, 4, "hot experts"),
]


@pytest.mark.parametrize("path", ["grouped", "route_direct"])
@pytest.mark.parametrize("T,H,I,E,k,tag", MX_CASES)
def test_mx_forward_parity(T, H, I, E, k, tag, path):
    say(f"mx {tag} {path}: T={T} H={H} I={I} E={E} k={k}")
    a = random_activations(T, H, E, seed=400 + T)
    lg = a["logits"]
    if tag == "hot experts":
        lg = lg.copy()
        lg[:, :k] += 50.0
    w = random_weights(E, H, I, "fp8_mx32", seed=401 + I)
    got, ref = _layer(a["x"], lg, k, w, path=path)
    check_out(got, ref, "fp8", f"{tag} {path}")


_DECODE_W = {}


def _decode_weights(H, I, E):
    """One MX weight set per decode shape, kept while consecutive cases use it."""
    if (H, I, E) not in _DECODE_W:
        _DECODE_W.clear()
        w = random_weights(E, H, I, "fp8_mx32", seed=460 + I)
        _DECODE_W[(H, I, E)] = (w, weights_dev(w, "fp8_mx32"))
    return _DECODE_W[(H, I, E)]


MX_DECODE = [(H, I, B) for H, I in ((2048, 768), (4096, 512)) for B in range(1, 9)]


@pytest.mark.parametrize("H,I,B", MX_DECODE)
def test_mx_route_direct_decode(H, I, B):
    """Route-direct MX at decode batches B = 1..8, E=128, top-8 (the shapes of the bf16 and
    blockwise decode layers): every launch shape the batch sizes select (row splits, waves per
    workgroup, Down K parts), the whole output against the oracle."""
    E, k = 128, 8
    w, (pw, sc) = _decode_weights(H, I, E)
    a = random_activations(B, H, E, seed=470 + B)
    li = moe.forward_launch_info(B, H, I, E, k, "fp8_mx32", "route_direct")
    say(f"mx route-direct decode B={B} H={H} I={I}: {li}")
    r = moe.route(torch.from_numpy(a["logits"]).to(DEV), k)
    out = moe.forward(bf16_dev(a["x"]), r, pw, quant="fp8_mx32", scales=sc, path="route_direct")
    torch.cuda.synchronize()
    ref_r = oracle.route(a["logits"], k)
    check_routing(routes_np(r), ref_r)
    check_out(out.float().cpu().numpy(), oracle_out(a["x"], ref_r, w, "fp8_mx32"), "fp8",
              f"mx decode B={B}")


@pytest.mark.parametrize("B", [1, 4])
def test_mx_decode_forward_folded_routing(B):
    """moe_decode_forward in MX: the routing taken inside the Gate/Up kernel from host logits."""
    H, I, E, k = 2048, 768, 128, 8
    w, (pw, sc) = _decode_weights(H, I, E)
    a = random_activations(B, H, E, seed=480 + B)
    say(f"mx decode_forward B={B}")
    out, r = moe.decode_forward(torch.from_numpy(a["logits"]).to(DEV), bf16_dev(a["x"]), k, pw,
                                quant="fp8_mx32", scales=sc, path="route_direct")
    torch.cuda.synchronize()
    ref_r = oracle.route(a["logits"], k)
    assert np.array_equal(r.topk_ids.cpu().numpy().reshape(B, k), ref_r["topk_ids"])
    check_out(out.float().cpu().numpy(), oracle_out(a["x"], ref_r, w, "fp8_mx32"), "fp8",
              f"mx decode_forward B={B}")


def test_mx_prefill_whole_output():
    """The blockwise prefill layer's shape (T=4096, H=4096, I=512, E=128, top-8) in MX: the
    whole output against the oracle."""
    T, H, I, E, k = 4096, 4096, 512, 128, 8
    say(f"mx prefill T={T} H={H} I={I} E={E} k={k}, whole output")
    a = random_activations(T, H, E, seed=410)
    w = random_weights(E, H, I, "fp8_mx32", seed=411)
    got, ref = _layer(a["x"], a["logits"], k, w)
    check_out(got, ref, "fp8", "mx prefill whole output")


@pytest.mark.parametrize("path", ["grouped", "route_direct"])
def test_mx_wide_scale_range(path):
    """Per-32 magnitudes spanning 1e4 along K in x and in the weights: every MX block takes a very
    different E8M0 byte, so a scale applied to the wrong 32 values shows."""
    T, H, I, E, k = 29, 512, 256, 4, 2
    a = random_activations(T, H, E, seed=420)
    fx = np.tile(np.array([1e-2, 1.0, 1e2, 1e-1, 10.0, 3e-2, 30.0, 0.3], np.float32), H // 256)
    x_bits = to_bf16_bits(bf16_bits_to_f32(a["x"]) * np.repeat(fx, 32)[None, :])
    gw = np.array([0.1, 10.0, 1.0, 0.3, 3.0, 1.0, 10.0, 0.1], np.float32)
    wgu = _normal_per_expert((E, H, 2 * I), 23, 0, 0.02) * np.repeat(np.tile(gw, H // 256), 32)[None, :, None]
    wd = _normal_per_expert((E, I, H), 23, 1, 0.02) * np.repeat(np.tile(gw, I // 256), 32)[None, :, None]
    qgu, sgu = quantise_weight_mx32(wgu)
    qd, sd = quantise_weight_mx32(wd)
    w = dict(w_gate_up=qgu, w_down=qd, s_gate_up=sgu, s_down=sd)
    got, ref = _layer(x_bits, a["logits"], k, w, path=path)
    check_out(got, ref, "fp8", f"mx wide scale range {path}")


@pytest.mark.parametrize("path", ["grouped", "route_direct"])
def test_mx_expert_slices_accumulate(path):
    T, H, I, E, k = 40, 256, 256, 8, 2
    a = random_activations(T, H, E, seed=430)
    w = random_weights(E, H, I, "fp8_mx32", seed=431)
    r = moe.route(torch.from_numpy(a["logits"]).to(DEV), k)
    ref_r = oracle.route(a["logits"], k)
    shared = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    total = np.zeros((T, H))
    for e0, n in ((0, 3), (3, 5)):
        ws = {key: (None if w[key] is None else np.ascontiguousarray(w[key][e0:e0 + n])) for key in w}
        pw, sc = weights_dev(ws, "fp8_mx32")
        moe.forward(bf16_dev(a["x"]), r, pw, quant="fp8_mx32", scales=sc, out=shared, expert_begin=e0,
                    num_experts=n, accumulate=True, path=path)
        total += oracle.forward(a["x"], ref_r["topk_ids"], ref_r["topk_weights"], ws["w_gate_up"], ws["w_down"],
                                quant="fp8_mx32", s_gate_up=ws["s_gate_up"], s_down=ws["s_down"],
                                expert_begin=e0)
    torch.cuda.synchronize()
    check_out(shared.float().cpu().numpy(), total, "fp8", f"mx slices accumulated {path}")


def test_mx_scale_packing_layout():
    """moe_pack_mx_scales against the documented order, computed here with numpy: per expert
    [N/32][K/256][64 lanes] dwords, lane 32hh + j, byte u = scale of packed row 32rb + j and K block
    8g + 2u + hh."""
    E, H, I = 2, 512, 256
    rng = np.random.default_rng(440)
    s_gu = rng.integers(100, 140, size=(E, H // 32, 2 * I), dtype=np.uint8)
    s_d = rng.integers(100, 140, size=(E, I // 32, H), dtype=np.uint8)
    pgu, pd = moe.pack_mx_scales(torch.from_numpy(s_gu).to(DEV), torch.from_numpy(s_d).to(DEV))
    torch.cuda.synchronize()

    def gate_up_col(P):   # packed row -> source column (gate c, up I + c)
        G, p = P >> 6, P & 63
        f, a_, hh, b = p >> 5, (p >> 3) & 3, (p >> 2) & 1, p & 3
        c = 32 * G + 16 * hh + 4 * a_ + b
        return c if f == 0 else I + c

    def down_col(P):
        G, p = P >> 6, P & 63
        f, a_, hh, b = p >> 5, (p >> 3) & 3, (p >> 2) & 1, p & 3
        return 64 * G + 32 * hh + 16 * f + 4 * a_ + b

    for src, got, K, N, colf in ((s_gu, pgu, H, 2 * I, gate_up_col), (s_d, pd, I, H, down_col)):
        ref = np.empty((E, N // 32, K // 256, 64, 4), np.uint8)
        for rb in range(N // 32):
            for lane in range(64):
                col = colf(32 * rb + (lane & 31))
                for g in range(K // 256):
                    for u in range(4):
                        ref[:, rb, g, lane, u] = src[:, 8 * g + 2 * u + (lane >> 5), col]
        assert np.array_equal(got.cpu().numpy().reshape(-1), ref.reshape(-1))


def test_mx_two_runs_bitwise_equal():
    T, H, I, E, k = 300, 512, 256, 8, 2
    a = random_activations(T, H, E, seed=450)
    w = random_weights(E, H, I, "fp8_mx32", seed=451)
    pw, sc = weights_dev(w, "fp8_mx32")
    r = moe.route(torch.from_numpy(a["logits"]).to(DEV), k)
    o1 = moe.forward(bf16_dev(a["x"]), r, pw, quant="fp8_mx32", scales=sc)
    o2 = moe.forward(bf16_dev(a["x"]), r, pw, quant="fp8_mx32", scales=sc)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
