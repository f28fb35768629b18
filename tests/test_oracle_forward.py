"""Pins of the oracle's layer output (CPU only).

Each pin reaches the same numbers by another route than the oracle's C code:
  * a hand-evaluated example (tests/golden/hand_example.json);
  * E=1: the plain SwiGLU FFN in torch float64 matrix form;
  * k=E with equal logits: the mean of all experts' FFNs;
  * brute force: every expert evaluated densely for every token with torch,
    then masked by the routing and weighted (no permutation anywhere);
  * FP8: the same dense formulation on tensors quantised with torch's own e4m3
    cast, per-tensor and 128x128 blockwise.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import (bf16_bits_to_f32, random_activations, random_weights,
                       to_bf16_bits)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")


def dense_experts(a, wgu, wd):
    """a [T,H] f64, wgu [E,H,2I] f64, wd [E,I,H] f64 -> Y [T,E,H] (every expert)."""
    I = wd.shape[1]
    gu = torch.einsum("th,ehn->ten", a, wgu)
    h = F.silu(gu[..., :I]) * gu[..., I:]
    return torch.einsum("tei,eih->teh", h, wd)


def combine_dense(Y, ids, w):
    T, E, H = Y.shape
    mask = torch.zeros(T, E, dtype=torch.float64)
    mask.scatter_(1, torch.from_numpy(ids.astype(np.int64)), torch.from_numpy(w.astype(np.float64)))
    return torch.einsum("te,teh->th", mask, Y)


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_golden_hand_example_forward():
    g = json.load(open(GOLDEN))
    x = to_bf16_bits(np.array(g["x"], np.float32))
    assert np.array_equal(bf16_bits_to_f32(x), np.array(g["x"], np.float32))
    wgu = to_bf16_bits(np.array(g["w_gate_up"], np.float32))
    wd = to_bf16_bits(np.array(g["w_down"], np.float32))
    r = oracle.route(np.array(g["logits"], np.float32), g["k"])
    out = oracle.forward(x, r["topk_ids"], r["topk_weights"], wgu, wd)
    ex = np.array(g["expected"]["out"])
    assert np.max(np.abs(out - ex)) <= g["expected"]["tolerance_out"]


def test_single_expert_is_plain_swiglu_ffn():
    T, H, I = 9, 64, 32
    a = random_activations(T, H, 1, 21)
    w = random_weights(1, H, I, "bf16", 22)
    r = oracle.route(a["logits"], 1)
    out = oracle.forward(a["x"], r["topk_ids"], r["topk_weights"], w["w_gate_up"], w["w_down"])
    x = torch.from_numpy(bf16_bits_to_f32(a["x"])).double()
    wg = torch.from_numpy(bf16_bits_to_f32(w["w_gate_up"][0])).double()
    wdn = torch.from_numpy(bf16_bits_to_f32(w["w_down"][0])).double()
    ref = (F.silu(x @ wg[:, :I]) * (x @ wg[:, I:])) @ wdn
    assert np.max(np.abs(out - ref.numpy())) <= 1e-12


def test_all_experts_equal_gates_is_expert_mean():
    T, H, I, E = 6, 32, 16, 8
    a = random_activations(T, H, E, 23)
    w = random_weights(E, H, I, "bf16", 24)
    lg = np.zeros((T, E), np.float32)
    r = oracle.route(lg, E)
    out = oracle.forward(a["x"], r["topk_ids"], r["topk_weights"], w["w_gate_up"], w["w_down"])
    x = torch.from_numpy(bf16_bits_to_f32(a["x"])).double()
    Y = dense_experts(x, torch.from_numpy(bf16_bits_to_f32(w["w_gate_up"])).double(),
                      torch.from_numpy(bf16_bits_to_f32(w["w_down"])).double())
    assert np.max(np.abs(out - Y.mean(dim=1).numpy())) <= 1e-12


@pytest.mark.parametrize("T,H,I,E,k,seed", [(12, 32, 16, 6, 3, 30), (20, 64, 32, 16, 8, 31),
                                            (5, 16, 8, 3, 1, 32)])
def test_brute_force_dense_masked(T, H, I, E, k, seed):
    a = random_activations(T, H, E, seed)
    w = random_weights(E, H, I, "bf16", seed + 100)
    r = oracle.route(a["logits"], k)
    out = oracle.forward(a["x"], r["topk_ids"], r["topk_weights"], w["w_gate_up"], w["w_down"])
    x = torch.from_numpy(bf16_bits_to_f32(a["x"])).double()
    Y = dense_experts(x, torch.from_numpy(bf16_bits_to_f32(w["w_gate_up"])).double(),
                      torch.from_numpy(bf16_bits_to_f32(w["w_down"])).double())
    ref = combine_dense(Y, r["topk_ids"], r["topk_weights"]).numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12
    # a token subset gives the same rows
    sub = np.array([T - 1, 0, T // 2], np.int32)
    out_s = oracle.forward(a["x"], r["topk_ids"], r["topk_weights"], w["w_gate_up"], w["w_down"],
                           tokens=sub)
    assert np.array_equal(out_s, out[sub])


def torch_e4m3(v):
    return torch.clamp(v.float(), -448, 448).to(torch.float8_e4m3fn).double()


def torch_scale(amax):
    amax = torch.as_tensor(amax, dtype=torch.float32)
    return torch.where(amax > 0, amax / torch.tensor(448.0, dtype=torch.float32),
                       torch.tensor(1.0, dtype=torch.float32))


@pytest.mark.parametrize("E,k", [(1, 1), (6, 3)])
def test_fp8_per_tensor_dense_reformulation(E, k):
    T, H, I = 10, 64, 32
    a = random_activations(T, H, E, 40 + E)
    w = random_weights(E, H, I, "fp8_per_tensor", 41 + E)
    r = oracle.route(a["logits"], k)
    out = oracle.forward(a["x"], r["topk_ids"], r["topk_weights"], w["w_gate_up"], w["w_down"],
                         quant="fp8_per_tensor", s_gate_up=w["s_gate_up"], s_down=w["s_down"])
    x = torch.from_numpy(bf16_bits_to_f32(a["x"]))
    sx = torch_scale(x.abs().max())
    xa = torch_e4m3(x / sx) * sx.double()
    wgu = (torch.from_numpy(w["w_gate_up"]).view(torch.float8_e4m3fn).double()
           * torch.from_numpy(w["s_gate_up"]).double()[:, None, None])
    wdn = (torch.from_numpy(w["w_down"]).view(torch.float8_e4m3fn).double()
           * torch.from_numpy(w["s_down"]).double()[:, None, None])
    gu = torch.einsum("th,ehn->ten", xa, wgu)
    h = (F.silu(gu[..., :I]) * gu[..., I:]).float()          # [T,E,I] fp32
    ids = torch.from_numpy(r["topk_ids"].astype(np.int64))
    h_routes = torch.gather(h, 1, ids[:, :, None].expand(T, k, I))   # the routed rows only
    sh = torch_scale(h_routes.abs().max())
    hq = torch_e4m3(h_routes / sh) * sh.double()                     # [T,k,I]
    y = torch.einsum("tji,tjih->tjh", hq, wdn[ids])
    ref = (y * torch.from_numpy(r["topk_weights"]).double()[:, :, None]).sum(dim=1)
    assert np.max(np.abs(out - ref.numpy())) <= 1e-12


def test_fp8_block128_dense_reformulation():
    T, H, I, E, k = 7, 256, 256, 4, 2
    a = random_activations(T, H, E, 50)
    w = random_weights(E, H, I, "fp8_block128", 51)
    r = oracle.route(a["logits"], k)
    out = oracle.forward(a["x"], r["topk_ids"], r["topk_weights"], w["w_gate_up"], w["w_down"],
                         quant="fp8_block128", s_gate_up=w["s_gate_up"], s_down=w["s_down"])
    x = torch.from_numpy(bf16_bits_to_f32(a["x"])).reshape(T, H // 128, 128)
    sx = torch_scale(x.abs().amax(dim=2))
    xa = (torch_e4m3(x / sx[:, :, None]) * sx.double()[:, :, None]).reshape(T, H)

    def deq(q, s):
        Ee, K, N = q.shape
        v = torch.from_numpy(q).view(torch.float8_e4m3fn).double().reshape(Ee, K // 128, 128, N // 128, 128)
        return (v * torch.from_numpy(s).double()[:, :, None, :, None]).reshape(Ee, K, N)

    wgu, wdn = deq(w["w_gate_up"], w["s_gate_up"]), deq(w["w_down"], w["s_down"])
    gu = torch.einsum("th,ehn->ten", xa, wgu)
    h = (F.silu(gu[..., :I]) * gu[..., I:]).float().reshape(T, E, I // 128, 128)
    sh = torch_scale(h.abs().amax(dim=3))
    hq = (torch_e4m3(h / sh[..., None]) * sh.double()[..., None]).reshape(T, E, I)
    Y = torch.einsum("tei,eih->teh", hq, wdn)
    ref = combine_dense(Y, r["topk_ids"], r["topk_weights"]).numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_fp8_mx32_dense_reformulation():
    """MX FP8: weights as codes times 2^(b-127) per 32 rows of K and column; x per token and h per
    route row quantised per 32 channels with the E8M0 rule (torch's frexp and e4m3 cast); the
    whole layer densely in torch."""
    T, H, I, E, k = 6, 128, 96, 4, 2
    a = random_activations(T, H, E, 52)
    w = random_weights(E, H, I, "fp8_mx32", 53)
    r = oracle.route(a["logits"], k)
    out = oracle.forward(a["x"], r["topk_ids"], r["topk_weights"], w["w_gate_up"], w["w_down"],
                         quant="fp8_mx32", s_gate_up=w["s_gate_up"], s_down=w["s_down"])

    def mx(v):   # [..., 32] fp32 -> dequantised fp64
        amax = v.abs().amax(dim=-1)
        _, ex = torch.frexp(amax)
        b = torch.where(amax > 0, (ex - 9 + 127).clamp(0, 254), torch.zeros_like(ex)).double()
        sc = torch.pow(2.0, b - 127)
        return torch_e4m3((v.double() / sc[..., None]).float()) * sc[..., None]

    x = torch.from_numpy(bf16_bits_to_f32(a["x"])).reshape(T, H // 32, 32)
    xa = mx(x).reshape(T, H)

    def deq(q, s):
        Ee, K, N = q.shape
        v = torch.from_numpy(q).view(torch.float8_e4m3fn).double().reshape(Ee, K // 32, 32, N)
        return (v * torch.pow(2.0, torch.from_numpy(s).double() - 127)[:, :, None, :]).reshape(Ee, K, N)

    wgu, wdn = deq(w["w_gate_up"], w["s_gate_up"]), deq(w["w_down"], w["s_down"])
    gu = torch.einsum("th,ehn->ten", xa, wgu)
    h = (F.silu(gu[..., :I]) * gu[..., I:]).float().reshape(T, E, I // 32, 32)
    hq = mx(h).reshape(T, E, I)
    Y = torch.einsum("tei,eih->teh", hq, wdn)
    ref = combine_dense(Y, r["topk_ids"], r["topk_weights"]).numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_quantisation_matters():
    """The FP8 oracle is not the bf16 oracle on dequantised weights: dropping the
    activation quantisation moves the result by far more than the FP8 parity
    tolerance, so the emulated quantisation is load-bearing."""
    T, H, I, E, k = 16, 256, 128, 4, 2
    a = random_activations(T, H, E, 60)
    w = random_weights(E, H, I, "fp8_block128", 61)
    r = oracle.route(a["logits"], k)
    q = oracle.forward(a["x"], r["topk_ids"], r["topk_weights"], w["w_gate_up"], w["w_down"],
                       quant="fp8_block128", s_gate_up=w["s_gate_up"], s_down=w["s_down"])
    x = torch.from_numpy(bf16_bits_to_f32(a["x"])).double()

    def deq(qq, s):
        Ee, K, N = qq.shape
        v = torch.from_numpy(qq).view(torch.float8_e4m3fn).double().reshape(Ee, K // 128, 128, N // 128, 128)
        return (v * torch.from_numpy(s).double()[:, :, None, :, None]).reshape(Ee, K, N)

    Y = dense_experts(x, deq(w["w_gate_up"], w["s_gate_up"]), deq(w["w_down"], w["s_down"]))
    plain = combine_dense(Y, r["topk_ids"], r["topk_weights"]).numpy()
    assert rel_l2(q, plain) > 1e-2


# ------------------------------------------------------ expert-parallel slice --
# A forward call may hold only experts [e0, e0 + n) (P3 Summary: the fast path
# preserves EP routing and shared output): routes to other experts contribute
# nothing and the per-tensor h scale covers the local routes only.

def _slice_w(w, e0, n):
    out = dict(w_gate_up=w["w_gate_up"][e0:e0 + n], w_down=w["w_down"][e0:e0 + n])
    for key in ("s_gate_up", "s_down"):
        out[key] = None if w[key] is None else np.ascontiguousarray(w[key][e0:e0 + n])
    return out


def test_ep_slices_brute_force_and_partition_bf16():
    T, H, I, E, k = 14, 32, 16, 8, 3
    a = random_activations(T, H, E, 60)
    w = random_weights(E, H, I, "bf16", 61)
    r = oracle.route(a["logits"], k)
    x = torch.from_numpy(bf16_bits_to_f32(a["x"])).double()
    Y = dense_experts(x, torch.from_numpy(bf16_bits_to_f32(w["w_gate_up"])).double(),
                      torch.from_numpy(bf16_bits_to_f32(w["w_down"])).double())
    full = oracle.forward(a["x"], r["topk_ids"], r["topk_weights"], w["w_gate_up"], w["w_down"])
    total = np.zeros_like(full)
    for e0, n in ((0, 3), (3, 4), (7, 1)):
        ws = _slice_w(w, e0, n)
        out = oracle.forward(a["x"], r["topk_ids"], r["topk_weights"], ws["w_gate_up"], ws["w_down"],
                             expert_begin=e0)
        local = (r["topk_ids"] >= e0) & (r["topk_ids"] < e0 + n)
        ref = combine_dense(Y, r["topk_ids"], np.where(local, r["topk_weights"], 0.0)).numpy()
        assert np.max(np.abs(out - ref)) <= 1e-12, (e0, n)
        total += out
    assert np.max(np.abs(total - full)) <= 1e-12


def test_ep_per_tensor_scale_covers_local_routes():
    T, H, I, E, k = 10, 64, 32, 6, 3
    e0, n = 2, 3
    a = random_activations(T, H, E, 62)
    w = random_weights(E, H, I, "fp8_per_tensor", 63)
    r = oracle.route(a["logits"], k)
    ws = _slice_w(w, e0, n)
    out = oracle.forward(a["x"], r["topk_ids"], r["topk_weights"], ws["w_gate_up"], ws["w_down"],
                         quant="fp8_per_tensor", s_gate_up=ws["s_gate_up"], s_down=ws["s_down"],
                         expert_begin=e0)
    x = torch.from_numpy(bf16_bits_to_f32(a["x"]))
    sx = torch_scale(x.abs().max())
    xa = torch_e4m3(x / sx) * sx.double()
    wgu = (torch.from_numpy(w["w_gate_up"]).view(torch.float8_e4m3fn).double()
           * torch.from_numpy(w["s_gate_up"]).double()[:, None, None])
    wdn = (torch.from_numpy(w["w_down"]).view(torch.float8_e4m3fn).double()
           * torch.from_numpy(w["s_down"]).double()[:, None, None])
    gu = torch.einsum("th,ehn->ten", xa, wgu)
    h = (F.silu(gu[..., :I]) * gu[..., I:]).float()
    ids = torch.from_numpy(r["topk_ids"].astype(np.int64))
    local = (ids >= e0) & (ids < e0 + n)
    h_routes = torch.gather(h, 1, ids[:, :, None].expand(T, k, I))
    sh = torch_scale(h_routes[local].abs().max())                     # local routes only
    hq = torch_e4m3(h_routes / sh) * sh.double()
    y = torch.einsum("tji,tjih->tjh", hq, wdn[ids])
    gw = torch.from_numpy(r["topk_weights"]).double() * local.double()
    ref = (y * gw[:, :, None]).sum(dim=1)
    assert np.max(np.abs(out - ref.numpy())) <= 1e-12
    # the scale differs from the whole layer's, so the slice is not a restriction of it
    assert local.any() and not local.all()


def test_ep_block128_partition_sums_to_layer():
    T, H, I, E, k = 6, 256, 256, 4, 2
    a = random_activations(T, H, E, 64)
    w = random_weights(E, H, I, "fp8_block128", 65)
    r = oracle.route(a["logits"], k)
    kw = dict(quant="fp8_block128")
    full = oracle.forward(a["x"], r["topk_ids"], r["topk_weights"], w["w_gate_up"], w["w_down"],
                          s_gate_up=w["s_gate_up"], s_down=w["s_down"], **kw)
    total = np.zeros_like(full)
    for e0, n in ((0, 1), (1, 3)):
        ws = _slice_w(w, e0, n)
        total += oracle.forward(a["x"], r["topk_ids"], r["topk_weights"], ws["w_gate_up"], ws["w_down"],
                                s_gate_up=ws["s_gate_up"], s_down=ws["s_down"], expert_begin=e0, **kw)
    assert np.max(np.abs(total - full)) <= 1e-12 * max(1.0, np.max(np.abs(full)))


def test_ep_slice_without_routes_is_zero():
    T, H, I, E, k = 5, 32, 16, 8, 2
    a = random_activations(T, H, E, 66)
    lg = a["logits"].copy()
    lg[:, :k] += 50.0                        # every token picks experts 0..k-1
    w = random_weights(E, H, I, "bf16", 67)
    r = oracle.route(lg, k)
    ws = _slice_w(w, 4, 3)
    out = oracle.forward(a["x"], r["topk_ids"], r["topk_weights"], ws["w_gate_up"], ws["w_down"],
                         expert_begin=4)
    assert np.array_equal(out, np.zeros_like(out))


@pytest.mark.parametrize("quant", ["bf16", "fp8_per_tensor", "fp8_block128", "fp8_mx32"])
def test_gate_up_h_dense_reformulation(quant):
    """oracle.gate_up_h: the SwiGLU output of each route, against torch's dense product of the
    activation (quantised with torch's own e4m3 cast for the FP8 formats) and every expert's
    Gate/Up weight, gathered at the routed (token, expert) pairs; a listed subset of routes
    returns exactly those rows."""
    T, H, I, E, k = 6, 256, 128, 5, 2
    a = random_activations(T, H, E, 60)
    w = random_weights(E, H, I, quant, 61)
    r = oracle.route(a["logits"], k)
    h = oracle.gate_up_h(a["x"], r["topk_ids"], w["w_gate_up"], quant, w["s_gate_up"])
    x = torch.from_numpy(bf16_bits_to_f32(a["x"]))
    if quant == "bf16":
        xa = x.double()
        wgu = torch.from_numpy(bf16_bits_to_f32(w["w_gate_up"])).double()
    else:
        q = torch.from_numpy(w["w_gate_up"]).view(torch.float8_e4m3fn).double()
        s = torch.from_numpy(w["s_gate_up"])
        if quant == "fp8_per_tensor":
            sx = torch_scale(x.abs().max())
            xa = torch_e4m3(x / sx) * sx.double()
            wgu = q * s.double()[:, None, None]
        elif quant == "fp8_block128":
            xb = x.reshape(T, H // 128, 128)
            sx = torch_scale(xb.abs().amax(dim=2))
            xa = (torch_e4m3(xb / sx[:, :, None]) * sx.double()[:, :, None]).reshape(T, H)
            wgu = (q.reshape(E, H // 128, 128, 2 * I // 128, 128)
                   * s.double()[:, :, None, :, None]).reshape(E, H, 2 * I)
        else:
            xb = x.reshape(T, H // 32, 32)
            amax = xb.abs().amax(dim=-1)
            _, ex = torch.frexp(amax)
            b = torch.where(amax > 0, (ex - 9 + 127).clamp(0, 254), torch.zeros_like(ex)).double()
            sc = torch.pow(2.0, b - 127)
            xa = (torch_e4m3((xb.double() / sc[..., None]).float()) * sc[..., None]).reshape(T, H)
            wgu = (q.reshape(E, H // 32, 32, 2 * I) * torch.pow(2.0, s.double() - 127)[:, :, None, :]).reshape(
                E, H, 2 * I)
    gu = torch.einsum("th,ehn->ten", xa, wgu)
    dense = (F.silu(gu[..., :I]) * gu[..., I:]).numpy()            # [T, E, I]
    ids = r["topk_ids"]
    ref = np.stack([dense[t, ids[t, j]] for t in range(T) for j in range(k)])
    assert np.max(np.abs(h - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
    sub = np.array([5, 0, 11], np.int32)
    assert np.array_equal(oracle.gate_up_h(a["x"], ids, w["w_gate_up"], quant, w["s_gate_up"], routes=sub),
                          h[sub])
