"""GPU parity of the MX training backward (moe_backward) against the oracle's
backward_mx ("[mxfp8 moe training] add per group blocked scale kernels":
Summary and stacked pull requests): the input gradient, the gates' gradient
and both weight gradients, each within the FP8 tolerance (rel-L2 2e-2, cosine
0.999); an expert without routes must get exact zeros; two calls give the same
bits.  Inputs are seeded: bf16 master weights, x, logits and the upstream
gradient dout."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, bf16_dev, check_out, check_routing, moe, oracle, random_activations, random_weights, \
    routes_np, say
from workloads import WORKLOADS, bf16_bits_to_f32, quantise_weight_mx32, random_upstream

pytestmark = pytest.mark.gpu


def _bwd(x_bits, lg, k, w, dout_bits):
    r = moe.route(torch.from_numpy(np.ascontiguousarray(lg)).to(DEV), k)
    tw = moe.prepare_mx_train_weights(bf16_dev(w["w_gate_up"]), bf16_dev(w["w_down"]))
    g = moe.backward(bf16_dev(x_bits), r, tw, bf16_dev(dout_bits))
    torch.cuda.synchronize()
    return r, {n: v.float().cpu().numpy() for n, v in g.items()}


def _compare(got, ref, tokens, experts, what):
    check_out(got["dx"][tokens], ref["dx"], "fp8", f"{what} dx")
    check_out(got["dgate"][tokens], ref["dgate"], "fp8", f"{what} dgate")
    check_out(got["dw_gate_up"][experts], ref["dw_gate_up"], "fp8", f"{what} dW_gate_up")
    check_out(got["dw_down"][experts], ref["dw_down"], "fp8", f"{what} dW_down")


CASES = [
    # (T, H, I, E, k, tag)
    (64, 256, 256, 4, 2, "small"),
    (100, 512, 256, 8, 4, "ragged segments"),
    (33, 256, 256, 1, 1, "E=1"),
    (40, 256, 512, 6, 6, "k=E, 2 Down column tiles"),
    (200, 256, 256, 16, 4, "hot experts, idle experts"),
    (300, 256, 768, 5, 2, "long route segments, I=768"),
]


@pytest.mark.parametrize("T,H,I,E,k,tag", CASES)
def test_backward_parity(T, H, I, E, k, tag):
    say(f"backward {tag}: T={T} H={H} I={I} E={E} k={k}")
    a = random_activations(T, H, E, seed=600 + T)
    lg = a["logits"]
    if tag.startswith("hot"):
        lg = lg.copy()
        lg[:, :k] += 50.0
    w = random_weights(E, H, I, "bf16", seed=601 + I)
    dout = random_upstream(T, H, 602 + E)
    r, got = _bwd(a["x"], lg, k, w, dout)
    ref_r = oracle.route(lg, k)
    check_routing(routes_np(r), ref_r)
    ref = oracle.backward_mx(a["x"], ref_r["topk_ids"], ref_r["topk_weights"], w["w_gate_up"], w["w_down"], dout)
    _compare(got, ref, np.arange(T), np.arange(E), tag)
    idle = np.setdiff1d(np.arange(E), ref_r["topk_ids"].ravel())
    if tag.startswith("hot"):
        assert idle.size > 0
    for e in idle:
        assert not got["dw_gate_up"][e].any() and not got["dw_down"][e].any(), f"expert {e} has no routes"


def test_backward_empty_batch_gives_zero_weight_gradients():
    E, H, I, k = 4, 256, 256, 2
    w = random_weights(E, H, I, "bf16", seed=611)
    r = moe.route(torch.empty((0, E), dtype=torch.float32, device=DEV), k)
    tw = moe.prepare_mx_train_weights(bf16_dev(w["w_gate_up"]), bf16_dev(w["w_down"]))
    out = {"dx": torch.empty((0, H), dtype=torch.bfloat16, device=DEV),
           "dgate": torch.empty((0, k), dtype=torch.float32, device=DEV),
           "dw_gate_up": torch.full((E, H, 2 * I), 7.0, dtype=torch.bfloat16, device=DEV),
           "dw_down": torch.full((E, I, H), 7.0, dtype=torch.bfloat16, device=DEV)}
    g = moe.backward(torch.empty((0, H), dtype=torch.bfloat16, device=DEV), r, tw,
                     torch.empty((0, H), dtype=torch.bfloat16, device=DEV), out=out)
    torch.cuda.synchronize()
    assert not g["dw_gate_up"].any().item() and not g["dw_down"].any().item()


def test_backward_two_calls_bitwise_equal():
    T, H, I, E, k = 96, 512, 256, 8, 2
    a = random_activations(T, H, E, seed=620)
    w = random_weights(E, H, I, "bf16", seed=621)
    dout = random_upstream(T, H, 622)
    r = moe.route(torch.from_numpy(a["logits"]).to(DEV), k)
    tw = moe.prepare_mx_train_weights(bf16_dev(w["w_gate_up"]), bf16_dev(w["w_down"]))
    x, d = bf16_dev(a["x"]), bf16_dev(dout)
    g1 = {n: v.clone() for n, v in moe.backward(x, r, tw, d).items()}
    g2 = moe.backward(x, r, tw, d)
    torch.cuda.synchronize()
    for n in g1:
        assert torch.equal(g1[n], g2[n]), n


def test_backward_prefill_shape_sampled():
    """The MX prefill layer's shape (T=4096, H=4096, I=512, E=128, top-8): the
    gradients of 16 tokens and of two experts (the busiest and the least busy
    with routes) against the oracle."""
    wl = WORKLOADS["prefill_fp8_mx"]
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    say(f"backward prefill shape: T={T} H={H} I={I} E={E} k={k}")
    a = random_activations(T, H, E, seed=630)
    w = random_weights(E, H, I, "bf16", seed=631)
    dout = random_upstream(T, H, 632)
    r, got = _bwd(a["x"], a["logits"], k, w, dout)
    ref_r = oracle.route(a["logits"], k)
    check_routing(routes_np(r), ref_r)
    counts = ref_r["expert_counts"]
    busy = int(np.argmax(counts))
    light = int(np.argmin(np.where(counts > 0, counts, counts.max() + 1)))
    tokens = np.linspace(0, T - 1, 16).astype(np.int32)
    experts = np.array([busy, light], np.int32)
    say(f"  experts {busy} ({counts[busy]} routes), {light} ({counts[light]} routes)")
    ref = oracle.backward_mx(a["x"], ref_r["topk_ids"], ref_r["topk_weights"], w["w_gate_up"], w["w_down"], dout,
                             tokens=tokens, experts=experts)
    _compare(got, ref, tokens, experts, "prefill shape")


def _slice(tw, ptr, nbytes):
    off = ptr - tw.buf.data_ptr()
    return tw.buf[off:off + nbytes]


def test_prepared_sets_match_the_forward_packing():
    """The one-pass preparation writes the same bytes as quantising with the input
    generator's MX rule and packing with moe_pack_weights / moe_pack_mx_scales:
    W_down along I as the forward packs it, and W_down^T along H packed as a
    Down matrix of K = H, N = I."""
    E, H, I = 4, 512, 256
    w = random_weights(E, H, I, "bf16", seed=640)
    tw = moe.prepare_mx_train_weights(bf16_dev(w["w_gate_up"]), bf16_dev(w["w_down"]))
    wd = bf16_bits_to_f32(w["w_down"])                                   # [E, I, H]
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    # W_down along I, as the forward's Down weights
    cd, sd = quantise_weight_mx32(wd)
    cg, sg = quantise_weight_mx32(bf16_bits_to_f32(w["w_gate_up"]))
    pw = moe.pack_weights(u8(cg), u8(cd), "fp8_mx32")
    _, psd = moe.pack_mx_scales(u8(sg), u8(sd))
    torch.cuda.synchronize()
    assert torch.equal(_slice(tw, tw.desc.down_k, E * I * H), pw.down.view(torch.uint8).reshape(-1))
    assert torch.equal(_slice(tw, tw.desc.down_k_scales, E * I * H // 32), psd.reshape(-1))
    # W_down^T along H: a Down matrix with K = H, N = I (shape (E, H'=I, I'=H) for the packers)
    ct, st = quantise_weight_mx32(np.ascontiguousarray(wd.transpose(0, 2, 1)))   # [E, H, I] along H
    dummy_gu = np.zeros((E, I, 2 * H), np.uint8)
    dummy_sg = np.zeros((E, I // 32, 2 * H), np.uint8)
    pt = moe.pack_weights(u8(dummy_gu), u8(ct), "fp8_mx32")
    _, pst = moe.pack_mx_scales(u8(dummy_sg), u8(st))
    torch.cuda.synchronize()
    assert torch.equal(_slice(tw, tw.desc.down_t, E * I * H), pt.down.view(torch.uint8).reshape(-1))
    assert torch.equal(_slice(tw, tw.desc.down_t_scales, E * I * H // 32), pst.reshape(-1))


@pytest.mark.parametrize("T,E,k", [(37, 16, 4), (5, 512, 8), (64, 8, 8)])
def test_route_backward_parity(T, E, k):
    """moe_route_backward against the oracle's softmax Jacobian, on a seeded
    upstream gradient of the gates and the oracle's own routing."""
    rng = np.random.default_rng(650 + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    g = rng.standard_normal((T, k)).astype(np.float32)
    r = moe.route(torch.from_numpy(lg).to(DEV), k)
    dl = moe.route_backward(r, torch.from_numpy(g).to(DEV))
    torch.cuda.synchronize()
    ref_r = oracle.route(lg, k)
    check_routing(routes_np(r), ref_r)
    ref = oracle.route_backward(ref_r["topk_ids"], ref_r["topk_weights"], g, E)
    got = dl.cpu().numpy()
    assert np.max(np.abs(got - ref)) <= 2e-6 * max(1.0, np.max(np.abs(ref)))
    mask = np.zeros((T, E), bool)
    np.put_along_axis(mask, ref_r["topk_ids"].astype(np.int64), True, axis=1)
    assert not got[~mask].any()


def test_backward_to_the_logits():
    """The layer's gate gradient taken to the logits, on the GPU end to end,
    against the oracle's chain (its own gate gradient, then its Jacobian)."""
    T, H, I, E, k = 96, 256, 256, 8, 2
    a = random_activations(T, H, E, seed=660)
    w = random_weights(E, H, I, "bf16", seed=661)
    dout = random_upstream(T, H, 662)
    r = moe.route(torch.from_numpy(a["logits"]).to(DEV), k)
    tw = moe.prepare_mx_train_weights(bf16_dev(w["w_gate_up"]), bf16_dev(w["w_down"]))
    g = moe.backward(bf16_dev(a["x"]), r, tw, bf16_dev(dout))
    dl = moe.route_backward(r, g["dgate"])
    torch.cuda.synchronize()
    ref_r = oracle.route(a["logits"], k)
    ref = oracle.backward_mx(a["x"], ref_r["topk_ids"], ref_r["topk_weights"], w["w_gate_up"], w["w_down"], dout)
    ref_dl = oracle.route_backward(ref_r["topk_ids"], ref_r["topk_weights"], ref["dgate"].astype(np.float32), E)
    check_out(dl.cpu().numpy(), ref_dl, "fp8", "dlogits")


def test_backward_graph_replay_bitwise_equal():
    """moe_backward captured in a HIP graph (it records no memset node) and replayed
    three times, with eager work between the replays: every replay equals the eager
    call bit for bit."""
    T, H, I, E, k = 128, 256, 256, 8, 4
    a = random_activations(T, H, E, seed=670)
    w = random_weights(E, H, I, "bf16", seed=671)
    dout = random_upstream(T, H, 672)
    r = moe.route(torch.from_numpy(a["logits"]).to(DEV), k)
    tw = moe.prepare_mx_train_weights(bf16_dev(w["w_gate_up"]), bf16_dev(w["w_down"]))
    x, d = bf16_dev(a["x"]), bf16_dev(dout)
    ws = torch.empty(moe.backward_workspace_size(T, H, I, E, k), dtype=torch.uint8, device=DEV)
    out = {"dx": torch.empty((T, H), dtype=torch.bfloat16, device=DEV),
           "dgate": torch.empty((T, k), dtype=torch.float32, device=DEV),
           "dw_gate_up": torch.empty((E, H, 2 * I), dtype=torch.bfloat16, device=DEV),
           "dw_down": torch.empty((E, I, H), dtype=torch.bfloat16, device=DEV)}
    moe.backward(x, r, tw, d, workspace=ws, out=out)
    torch.cuda.synchronize()
    eager = {n: v.clone() for n, v in out.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.backward(x, r, tw, d, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.backward(x, r, tw, d, workspace=ws, out=out)
    for i in range(3):
        for v in out.values():
            v.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in out:
            assert torch.equal(out[n], eager[n]), (i, n)
        moe.backward(x, r, tw, d, workspace=ws, out={n: torch.empty_like(v) for n, v in out.items()})
        torch.cuda.synchronize()


def test_prepared_forward_equals_the_classic_mx_forward():
    """The forward set of the preparation runs moe_forward to the same bits as the
    MX weights quantised with the input generator's rule and packed with
    moe_pack_weights / moe_pack_mx_scales."""
    T, H, I, E, k = 150, 512, 256, 8, 4
    a = random_activations(T, H, E, seed=680)
    w = random_weights(E, H, I, "bf16", seed=681)
    u8 = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(DEV)
    tw = moe.prepare_mx_train_weights(bf16_dev(w["w_gate_up"]), bf16_dev(w["w_down"]))
    cg, sg = quantise_weight_mx32(bf16_bits_to_f32(w["w_gate_up"]))
    cd, sd = quantise_weight_mx32(bf16_bits_to_f32(w["w_down"]))
    pw = moe.pack_weights(u8(cg), u8(cd), "fp8_mx32")
    ps = moe.pack_mx_scales(u8(sg), u8(sd))
    r = moe.route(torch.from_numpy(a["logits"]).to(DEV), k)
    x = bf16_dev(a["x"])
    got = moe.forward(x, r, tw.forward, quant="fp8_mx32", scales=tw.forward_scales, path="grouped")
    ref = moe.forward(x, r, pw, quant="fp8_mx32", scales=ps, path="grouped")
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert torch.equal(tw.forward.gate_up.reshape(-1), pw.gate_up.view(torch.uint8).reshape(-1))
    assert torch.equal(tw.forward_scales[0], ps[0].reshape(-1))
