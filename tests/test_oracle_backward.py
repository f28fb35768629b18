"""Pins of the oracle's layer backward (CPU only).

Each pin reaches the gradients by another route than the oracle's C code:
  * exact mode (no quantiser): torch's autograd through a dense float64 form of
    the layer (every expert evaluated for every token, masked by the routing
    and weighted) -- an independent chain rule;
  * MX mode: the MX training recipe written densely in torch, each operand
    quantised with torch's frexp and e4m3 cast along its product's reduction
    dimension (the weight gradients' operands along each expert's routes,
    zero-padded to 32);
  * subsets of tokens and experts equal the rows of the full result, and the
    MX gradients stay close to the exact ones while differing from them.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import bf16_bits_to_f32, random_activations, random_upstream, random_weights


def _inputs(T, H, I, E, k, seed, logits="normal"):
    a = random_activations(T, H, E, seed, logits=logits)
    w = random_weights(E, H, I, "bf16", seed + 1)
    r = oracle.route(a["logits"], k)
    dout = random_upstream(T, H, seed + 2)
    return a, w, r, dout


def _f64(bits):
    return torch.from_numpy(bf16_bits_to_f32(bits).astype(np.float64))


@pytest.mark.parametrize("T,H,I,E,k,seed", [(12, 64, 32, 4, 2, 1), (9, 48, 40, 5, 5, 2), (16, 32, 16, 1, 1, 3)])
def test_exact_backward_matches_autograd(T, H, I, E, k, seed):
    a, w, r, dout = _inputs(T, H, I, E, k, seed)
    g = oracle.backward_mx(a["x"], r["topk_ids"], r["topk_weights"], w["w_gate_up"], w["w_down"], dout,
                           exact=True)
    x = _f64(a["x"]).requires_grad_(True)
    wgu = _f64(w["w_gate_up"]).requires_grad_(True)
    wd = _f64(w["w_down"]).requires_grad_(True)
    gates = torch.from_numpy(r["topk_weights"].astype(np.float64)).requires_grad_(True)
    ids = torch.from_numpy(r["topk_ids"].astype(np.int64))
    gu = torch.einsum("th,ehn->ten", x, wgu)
    h = F.silu(gu[..., :I]) * gu[..., I:]
    Y = torch.einsum("tei,eih->teh", h, wd)                       # every expert
    Yr = torch.gather(Y, 1, ids[:, :, None].expand(T, k, H))      # the routed ones
    out = (gates[:, :, None] * Yr).sum(dim=1)
    (out * _f64(dout)).sum().backward()
    for name, ref in (("dx", x.grad), ("dgate", gates.grad), ("dw_gate_up", wgu.grad), ("dw_down", wd.grad)):
        ref = ref.numpy()
        err = np.max(np.abs(g[name] - ref)) / max(np.max(np.abs(ref)), 1e-300)
        assert err <= 1e-12, (name, err)


def _mx_last(v):
    """MX along the last dimension (a multiple of 32): fp32 values -> dequantised float64."""
    sh = v.shape
    b32 = v.float().reshape(*sh[:-1], sh[-1] // 32, 32)
    amax = b32.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)
    b = torch.where(amax > 0, (ex - 9 + 127).clamp(0, 254), torch.zeros_like(ex)).double()
    sc = torch.pow(2.0, b - 127)
    codes = torch.clamp(b32.double() / sc[..., None], -448, 448).float().to(torch.float8_e4m3fn).double()
    return (codes * sc[..., None]).reshape(sh)


def _mx_along(v, dim):
    return _mx_last(v.movedim(dim, -1)).movedim(-1, dim)


def _recipe(a, w, r, dout, T, H, I, E, k):
    """The MX training backward written densely in torch."""
    x32 = torch.from_numpy(bf16_bits_to_f32(a["x"]))
    wgu = torch.from_numpy(bf16_bits_to_f32(w["w_gate_up"]))
    wd = torch.from_numpy(bf16_bits_to_f32(w["w_down"]))
    do32 = torch.from_numpy(bf16_bits_to_f32(dout))
    ids = torch.from_numpy(r["topk_ids"].astype(np.int64))
    gates32 = torch.from_numpy(r["topk_weights"])
    xa = _mx_last(x32)
    wgK, wdK = _mx_along(wgu, 1), _mx_along(wd, 1)             # forward: along K
    wg2, wdH = _mx_last(wgu), _mx_last(wd)                      # input gradients: along 2I, along H
    gu = torch.einsum("th,ehn->ten", xa, wgK)                   # [T,E,2I]
    gur = torch.gather(gu, 1, ids[:, :, None].expand(T, k, 2 * I))
    g_, u_ = gur[..., :I], gur[..., I:]
    h32 = (F.silu(g_) * u_).float()
    hq = _mx_last(h32)
    y = torch.einsum("tji,tjin->tjn", hq, wdK[ids])
    dgate = (y * do32.double()[:, None, :]).sum(dim=2)
    dy32 = gates32[:, :, None] * do32[:, None, :]                # fp32 products
    dh = torch.einsum("tjn,tjin->tji", _mx_last(dy32), wdH[ids])
    sg = torch.sigmoid(g_)
    dgu = torch.cat([dh * u_ * sg * (1 + g_ * (1 - sg)), dh * g_ * sg], dim=2)
    dgu32 = dgu.float()
    da = torch.einsum("tjc,tjhc->tjh", _mx_last(dgu32), wg2[ids])
    dx = da.sum(dim=1)
    dwg = torch.zeros(E, H, 2 * I, dtype=torch.float64)
    dwd = torch.zeros(E, I, H, dtype=torch.float64)
    flat = ids.reshape(-1)
    for e in range(E):
        rr = torch.nonzero(flat == e).flatten()                  # ascending route order
        n = rr.numel()
        if n == 0:
            continue
        npad = (n + 31) // 32 * 32

        def col(m):                                             # [n, c] -> padded, quantised along routes
            z = torch.zeros(npad, m.shape[1], dtype=torch.float32)
            z[:n] = m
            return _mx_along(z, 0)

        xs = x32[rr // k]
        dwg[e] = col(xs).T @ col(dgu32.reshape(T * k, 2 * I)[rr])
        dwd[e] = col(h32.reshape(T * k, I)[rr]).T @ col(dy32.reshape(T * k, H)[rr])
    return {"dx": dx.numpy(), "dgate": dgate.numpy(), "dw_gate_up": dwg.numpy(), "dw_down": dwd.numpy()}


@pytest.mark.parametrize("T,H,I,E,k,seed", [(40, 128, 64, 4, 2, 11), (70, 64, 32, 3, 3, 12), (33, 96, 32, 1, 1, 13)])
def test_mx_backward_matches_torch_recipe(T, H, I, E, k, seed):
    a, w, r, dout = _inputs(T, H, I, E, k, seed)
    g = oracle.backward_mx(a["x"], r["topk_ids"], r["topk_weights"], w["w_gate_up"], w["w_down"], dout)
    ref = _recipe(a, w, r, dout, T, H, I, E, k)
    for name in ("dx", "dgate", "dw_gate_up", "dw_down"):
        err = np.max(np.abs(g[name] - ref[name])) / max(np.max(np.abs(ref[name])), 1e-300)
        assert err <= 1e-9, (name, err)


def test_mx_backward_close_to_exact_and_quantised():
    T, H, I, E, k = 48, 128, 64, 4, 2
    a, w, r, dout = _inputs(T, H, I, E, k, 21)
    q = oracle.backward_mx(a["x"], r["topk_ids"], r["topk_weights"], w["w_gate_up"], w["w_down"], dout)
    x = oracle.backward_mx(a["x"], r["topk_ids"], r["topk_weights"], w["w_gate_up"], w["w_down"], dout,
                           exact=True)
    for name in ("dx", "dgate", "dw_gate_up", "dw_down"):
        rl = np.linalg.norm(q[name] - x[name]) / np.linalg.norm(x[name])
        assert 1e-4 < rl < 0.15, (name, rl)


def test_backward_subsets_are_rows_of_the_whole():
    T, H, I, E, k = 30, 64, 32, 5, 2
    a, w, r, dout = _inputs(T, H, I, E, k, 31)
    full = oracle.backward_mx(a["x"], r["topk_ids"], r["topk_weights"], w["w_gate_up"], w["w_down"], dout)
    tok = np.array([29, 3, 11], np.int32)
    exps = np.array([4, 0], np.int32)
    sub = oracle.backward_mx(a["x"], r["topk_ids"], r["topk_weights"], w["w_gate_up"], w["w_down"], dout,
                             tokens=tok, experts=exps)
    assert np.array_equal(sub["dx"], full["dx"][tok])
    assert np.array_equal(sub["dgate"], full["dgate"][tok])
    assert np.array_equal(sub["dw_gate_up"], full["dw_gate_up"][exps])
    assert np.array_equal(sub["dw_down"], full["dw_down"][exps])


def test_backward_expert_without_routes_has_zero_weight_gradient():
    T, H, I, E, k = 8, 64, 32, 6, 1
    a, w, r, dout = _inputs(T, H, I, E, k, 41)
    used = set(r["topk_ids"].ravel().tolist())
    idle = [e for e in range(E) if e not in used]
    assert idle, "the seed leaves no expert idle"
    g = oracle.backward_mx(a["x"], r["topk_ids"], r["topk_weights"], w["w_gate_up"], w["w_down"], dout,
                           experts=np.array(idle, np.int32))
    assert not g["dw_gate_up"].any() and not g["dw_down"].any()


@pytest.mark.parametrize("T,E,k,seed", [(17, 8, 2, 51), (5, 16, 16, 52), (9, 4, 1, 53)])
def test_route_backward_matches_autograd(T, E, k, seed):
    """The gates' gradient taken to the logits equals torch's autograd through
    the softmax over the picked logits (ids fixed: the picks do not move under
    an infinitesimal change of the logits)."""
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    r = oracle.route(lg, k)
    g = rng.standard_normal((T, k)).astype(np.float32)
    got = oracle.route_backward(r["topk_ids"], r["topk_weights"], g, E)
    l = torch.from_numpy(lg.astype(np.float64)).requires_grad_(True)
    ids = torch.from_numpy(r["topk_ids"].astype(np.int64))
    w = torch.softmax(torch.gather(l, 1, ids), dim=1)
    (w * torch.from_numpy(g.astype(np.float64))).sum().backward()
    ref = l.grad.numpy()
    assert np.max(np.abs(got - ref)) <= 1e-6 * max(1.0, np.max(np.abs(ref)))
    # unpicked logits get nothing, and each row sums to zero (the softmax's invariance to a shift)
    mask = np.zeros((T, E), bool)
    np.put_along_axis(mask, r["topk_ids"].astype(np.int64), True, axis=1)
    assert not got[~mask].any()
    assert np.max(np.abs(got.sum(axis=1))) <= 1e-6
