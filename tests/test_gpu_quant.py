"""FP8 activation quantisation on the GPU, compared byte for byte.

A forward call leaves the codes and scales it quantised x into in its workspace
(moe_forward_workspace_views).  With bf16 input, s = amax/448 as a true fp32
division and q = e4m3(v / s) rounded to nearest even (per tensor, per token per
128 channels, or MX E8M0 per 32), the codes are fully determined, so they must
equal oracle.quantise_activations bit for bit, on the grouped path, the
route-direct path and the decode entry with the routing folded in.  The
Down-input (h) scales depend on the Gate/Up products, whose fp32 summation order
differs from the oracle's, so they are compared within 1e-3 relative (MX: the
same E8M0 byte unless h's amax lies within that of a power of two), and the
grouped path's h codes must round the same way for at least 99% of the values;
the others lie next to a rounding boundary (one code step apart) or next to
zero (within 0.05 units of the group's scale).
"""
import numpy as np
import pytest
import torch

from gpu_helpers import (DEV, bf16_dev, moe, oracle, random_activations, random_weights, say, weights_dev,
                         workload_dev, workload_inputs, workload_weights, WORKLOADS)

pytestmark = pytest.mark.gpu


def _mx_unpermute(b: np.ndarray) -> np.ndarray:
    """E8M0 bytes [rows, G] in the GEMM's order (group c at 8(c/8) + 4(c%2) + (c%8)/2) ->
    natural group order."""
    G = b.shape[1]
    c = np.arange(G)
    return b[:, 8 * (c // 8) + 4 * (c % 2) + (c % 8) // 2]


def _run(x_bits, lg, k, quant, path, dev_w, E, H, I, fused=False):
    pw, sc = dev_w
    T = x_bits.shape[0]
    p = moe.select_path(T, H, I, E, k, quant, path)
    ws = torch.zeros(moe.forward_workspace_size(T, H, I, E, k, quant, p), dtype=torch.uint8, device=DEV)
    x = bf16_dev(x_bits)
    lgd = torch.from_numpy(np.ascontiguousarray(lg)).to(DEV)
    if fused:
        moe.decode_forward(lgd, x, k, pw, quant=quant, scales=sc, path=p, workspace=ws)
    else:
        r = moe.route(lgd, k)
        moe.forward(x, r, pw, quant=quant, scales=sc, path=p, workspace=ws)
    torch.cuda.synchronize()
    return p, ws.cpu().numpy(), moe.forward_workspace_views(T, H, I, E, k, quant, p)


def _check_x(ws, v, x_bits, quant):
    T, H = x_bits.shape
    ref_q, ref_s = oracle.quantise_activations(x_bits, quant)
    got_q = ws[v["x_codes"]:v["x_codes"] + T * H].reshape(T, H)
    assert np.array_equal(got_q, ref_q), f"x codes differ in {np.count_nonzero(got_q != ref_q)} places"
    if quant == "fp8_per_tensor":
        got_s = ws[v["x_scales"]:v["x_scales"] + 4].view(np.float32)[0]
        assert got_s.view(np.uint32) == np.float32(ref_s).view(np.uint32), (got_s, ref_s)
    elif quant == "fp8_block128":
        got_s = ws[v["x_scales"]:v["x_scales"] + 4 * T * (H // 128)].view(np.float32).reshape(T, H // 128)
        assert np.array_equal(got_s.view(np.uint32), ref_s.view(np.uint32))
    else:
        got_s = _mx_unpermute(ws[v["x_scales"]:v["x_scales"] + T * (H // 32)].reshape(T, H // 32))
        assert np.array_equal(got_s, ref_s)


def _group_quant(h, quant, group):
    """The oracle's own quantiser over h (fp32) per group: (codes [R, I], scales)."""
    R, I = h.shape
    hf = h.astype(np.float32)
    codes = np.empty((R, I), np.uint8)
    if quant == "fp8_per_tensor":
        q, s = oracle.quantise_group(hf.ravel())
        return q.reshape(R, I), np.float32(s)
    scales = np.empty((R, I // group), np.uint8 if quant == "fp8_mx32" else np.float32)
    for r in range(R):
        for c in range(I // group):
            if quant == "fp8_mx32":
                q, b = oracle.quantise_group_mx(hf[r, c * group:(c + 1) * group])
                scales[r, c] = b
            else:
                q, s = oracle.quantise_group(hf[r, c * group:(c + 1) * group])
                scales[r, c] = s
            codes[r, c * group:(c + 1) * group] = q
    return codes, scales


def _check_h(ws, v, h_ref, quant, path):
    R, I = h_ref.shape
    group = {"fp8_per_tensor": I, "fp8_block128": 128, "fp8_mx32": 32}[quant]
    ref_q, ref_s = _group_quant(h_ref, quant, group)
    if quant == "fp8_per_tensor":
        got_s = ws[v["h_scales"]:v["h_scales"] + 4].view(np.float32)[0]
        assert abs(got_s / ref_s - 1) <= 1e-3, (got_s, ref_s)
    elif quant == "fp8_block128":
        got_s = ws[v["h_scales"]:v["h_scales"] + 4 * R * (I // 128)].view(np.float32).reshape(R, I // 128)
        assert np.max(np.abs(got_s / ref_s - 1)) <= 1e-3
    else:
        got_s = _mx_unpermute(ws[v["h_scales"]:v["h_scales"] + R * (I // 32)].reshape(R, I // 32))
        amax = np.abs(h_ref.reshape(R, I // 32, 32)).max(axis=2)
        near = np.abs(np.log2(np.maximum(amax, 1e-30)) - np.round(np.log2(np.maximum(amax, 1e-30)))) < 2e-3
        assert np.all((got_s == ref_s) | (near & (np.abs(got_s.astype(int) - ref_s.astype(int)) <= 1)))
    if path != "grouped":
        assert v["h_codes"] is None
        return
    got_q = ws[v["h_codes"]:v["h_codes"] + R * I].reshape(R, I)
    same = got_q == ref_q
    mag_g, mag_r = got_q.astype(int) & 0x7F, ref_q.astype(int) & 0x7F
    sign_ok = ((got_q ^ ref_q) & 0x80 == 0) | ((mag_g <= 1) & (mag_r <= 1))
    # codes in units of their group's scale: next to zero the fp32 accumulation error of the
    # Gate/Up sums (about 1e-5 of the group's largest |h| over K = 1024) spans several
    # subnormal e4m3 steps, so there a difference up to 0.05 units (1.1e-4 of the amax) passes
    lut = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    near = np.abs(lut[got_q] - lut[ref_q]) <= 0.05
    assert np.mean(same) >= 0.99, np.mean(same)
    assert np.all(same | ((np.abs(mag_g - mag_r) <= 1) & sign_ok) | near)


CASES = [
    # (T, H, I, E, k, quant, path, fused)
    (150, 1024, 256, 16, 4, "fp8_per_tensor", "grouped", False),
    (3, 1024, 256, 16, 4, "fp8_per_tensor", "route_direct", False),
    (3, 1024, 256, 16, 4, "fp8_per_tensor", "route_direct", True),
    (150, 1024, 256, 16, 4, "fp8_block128", "grouped", False),
    (3, 1024, 256, 16, 4, "fp8_block128", "route_direct", False),
    (3, 1024, 256, 16, 4, "fp8_block128", "route_direct", True),
    (150, 1024, 256, 16, 4, "fp8_mx32", "grouped", False),
    (3, 1024, 256, 16, 4, "fp8_mx32", "route_direct", False),
    (3, 1024, 256, 16, 4, "fp8_mx32", "route_direct", True),
]


@pytest.mark.parametrize("T,H,I,E,k,quant,path,fused", CASES)
def test_quantised_activations_bytes(T, H, I, E, k, quant, path, fused):
    say(f"quant bytes {quant} {path}{' fused' if fused else ''}: T={T} H={H} I={I} E={E} k={k}")
    a = random_activations(T, H, E, seed=500 + T + E)
    w = random_weights(E, H, I, quant, seed=501 + I)
    p, ws, v = _run(a["x"], a["logits"], k, quant, path, weights_dev(w, quant), E, H, I, fused)
    _check_x(ws, v, a["x"], quant)
    ref_r = oracle.route(a["logits"], k)
    rows = ref_r["perm"] if p == "grouped" else None    # h rows: sorted order, or route order
    h_ref = oracle.gate_up_h(a["x"], ref_r["topk_ids"], w["w_gate_up"], quant, w["s_gate_up"], routes=rows)
    _check_h(ws, v, h_ref, quant, p)


@pytest.mark.parametrize("name,B,path", [("decode_fp8_tensor", 4, "route_direct"),
                                         ("decode_fp8_tensor", 8, "grouped"),
                                         ("prefill_fp8_block", None, "grouped")])
def test_quantised_x_bytes_full_size(name, B, path):
    """The x codes and scales at the benchmarked shapes (per-tensor decode, blockwise prefill)."""
    wl = WORKLOADS[name]
    a = workload_inputs(name, batch=B)
    T = a["x"].shape[0]
    say(f"quant bytes {name} T={T} {path}")
    p, ws, v = _run(a["x"], a["logits"], wl.k, wl.quant, path, workload_dev(name), wl.E, wl.H, wl.I)
    _check_x(ws, v, a["x"], wl.quant)
    if T <= 8:   # the decode batch's h is small enough for the oracle
        ref_r = oracle.route(a["logits"], wl.k)
        rows = ref_r["perm"] if p == "grouped" else None
        h_ref = oracle.gate_up_h(a["x"], ref_r["topk_ids"], workload_weights(name)["w_gate_up"], wl.quant,
                                 workload_weights(name)["s_gate_up"], routes=rows)
        _check_h(ws, v, h_ref, wl.quant, p)


def test_quantised_x_bytes_mx_prefill_shape():
    T, H, I, E, k = 4096, 4096, 512, 128, 8
    a = random_activations(T, H, E, seed=410)
    w = random_weights(E, H, I, "fp8_mx32", seed=411)
    p, ws, v = _run(a["x"], a["logits"], k, "fp8_mx32", "grouped", weights_dev(w, "fp8_mx32"), E, H, I)
    _check_x(ws, v, a["x"], "fp8_mx32")
