"""The C-ABI library loads, exports every entry point include/moe.h declares,
and rejects bad arguments on the host before any GPU call (CPU only)."""
import ctypes
import os
import re

import pytest
import torch

import routing_grouped_expert_index_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = moe.lib()
    names = header_functions()
    assert set(moe.EXPORTED) <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_select_path_rules():
    # route-direct while T*k <= 3E/4 and T <= 16 (the measured crossover), prefill goes grouped
    assert moe.select_path(1, 2048, 768, 128, 8) == "route_direct"
    assert moe.select_path(4, 2048, 768, 128, 8) == "route_direct"
    assert moe.select_path(12, 2048, 768, 128, 8) == "route_direct"     # 96 routes = 3E/4
    assert moe.select_path(13, 2048, 768, 128, 8) == "grouped"
    assert moe.select_path(4, 4096, 192, 192, 8, "fp8_per_tensor") == "route_direct"
    assert moe.select_path(16, 4096, 192, 192, 8, "fp8_per_tensor") == "route_direct"
    assert moe.select_path(17, 4096, 192, 192, 8, "fp8_per_tensor") == "grouped"   # past 16 tokens
    assert moe.select_path(8192, 2048, 768, 128, 8) == "grouped"
    assert moe.select_path(64, 256, 512, 16, 8) == "grouped"
    assert moe.select_path(1, 2048, 768, 128, 8, "bf16", "grouped") == "grouped"
    # MX FP8 follows the same rule (H and I multiples of 256, I <= 2048 on route-direct)
    assert moe.select_path(1, 2048, 768, 128, 8, "fp8_mx32") == "route_direct"
    assert moe.select_path(13, 2048, 768, 128, 8, "fp8_mx32") == "grouped"
    assert moe.select_path(1, 2048, 768, 128, 8, "fp8_mx32", "route_direct") == "route_direct"
    assert moe.select_path(1, 2048, 4096, 128, 8, "fp8_mx32") == "grouped"      # I past 2048 bytes
    with pytest.raises(moe.MoeError):
        moe.select_path(1, 2048, 4096, 128, 8, "fp8_mx32", "route_direct")
    with pytest.raises(moe.MoeError):
        moe.select_path(64, 2048, 192, 128, 8, "fp8_mx32")
    assert moe.select_path(64, 2048, 768, 128, 8, "bf16", "route_direct") == "route_direct"
    # H a multiple of 64 (not of 128) for bf16 and per-tensor FP8
    assert moe.select_path(1, 2112, 768, 128, 8) == "route_direct"
    assert moe.select_path(512, 2112, 768, 128, 8, "fp8_per_tensor") == "grouped"


@pytest.mark.parametrize("args,code", [
    ((1, 2048, 768, 4, 8, "bf16", "auto"), -1),      # k > E
    ((1, 2048, 768, 600, 8, "bf16", "auto"), -1),    # E > 512
    ((1, 2000, 768, 128, 8, "bf16", "auto"), -2),    # H % 64
    ((1, 2112, 768, 128, 8, "fp8_block128", "auto"), -2),   # block128 needs H % 128
    ((1, 2048, 96, 128, 8, "bf16", "auto"), -2),     # I % 64
    ((1, 2048, 192, 128, 8, "fp8_block128", "auto"), -2),   # block128 needs I % 128
    ((1, 16384, 768, 128, 8, "bf16", "route_direct"), -2),  # route-direct shape limit
    ((-1, 2048, 768, 128, 8, "bf16", "auto"), -1),
])
def test_select_path_errors(args, code):
    with pytest.raises(moe.MoeError) as ei:
        moe.select_path(*args)
    assert ei.value.code == code
    assert moe.lib().moe_last_error().decode()


def test_workspace_sizes():
    g = moe.forward_workspace_size(8192, 2048, 768, 128, 8, "bf16", "grouped")
    # at least h (bf16) and y (bf16) of all routes
    assert g >= 8192 * 8 * (768 + 2048) * 2
    rd = moe.forward_workspace_size(4, 2048, 768, 128, 8, "bf16", "route_direct")
    assert 0 < rd < 1 << 20
    assert moe.forward_workspace_size(1, 2048, 768, 4, 8) == 0   # invalid -> 0
    assert moe.route_workspace_size(8192, 128, 8) > 0
    assert moe.route_workspace_size(4, 128, 8) == 0


def _packed(E, H, I, quant=0, tag=None, addr=4096):
    """A descriptor as moe_pack_weights fills it (fake device addresses)."""
    return moe._CPacked(addr, addr, E, H, I, quant, moe.PACKED_TAG if tag is None else tag)


@pytest.mark.skipif(torch.cuda.is_available(),
                    reason="passes fake device addresses; only run where no GPU can be reached")
def test_host_validation_before_any_launch():
    L = moe.lib()
    r = moe._CRoutes()
    # k > E is rejected on the host (no device pointer is touched)
    assert L.moe_route(None, 4, 4, 8, ctypes.byref(r), None, 0, None) == -1
    assert L.moe_route(None, 4, 8, 2, None, None, 0, None) == -1
    # null routes / null pointers / bad quant
    assert L.moe_forward(None, None, None, None, None, 2048, 768, 0, 0, None, 0, None) == -1
    r.T, r.E, r.k = 4, 128, 8
    assert L.moe_forward(None, ctypes.byref(r), None, None, None, 2048, 768, 0, 0, None, 0, None) == -1
    assert L.moe_forward(None, ctypes.byref(r), None, None, None, 2048, 768, 7, 0, None, 0, None) == -1
    # T = 0 is a valid empty call: nothing to do, no launch
    r.T = 0
    assert L.moe_forward(None, ctypes.byref(r), None, None, None, 2048, 768, 0, 0, None, 0, None) == 0
    # misaligned pointers are rejected
    r.T = 4
    r.topk_ids = r.topk_weights = r.expert_offsets = r.perm = 4096
    bad = ctypes.c_void_p(4096 + 8)
    good = ctypes.c_void_p(4096)
    w = _packed(128, 2048, 768)
    assert L.moe_forward(bad, ctypes.byref(r), ctypes.byref(w), None, good, 2048, 768, 0, 0, good, 1 << 30,
                         None) == -1
    # short workspace
    assert L.moe_forward(good, ctypes.byref(r), ctypes.byref(w), None, good, 2048, 768, 0, 0, good, 16,
                         None) == -3
    # fp8 needs scales
    w8 = _packed(128, 2048, 768, quant=1)
    assert L.moe_forward(good, ctypes.byref(r), ctypes.byref(w8), None, good, 2048, 768, 1, 0, good, 1 << 30,
                         None) == -1
    # expert slices: [expert_begin, expert_begin + num_experts) inside [0, E), accumulate 0 or 1
    for e0, n, acc in ((-1, 4, 0), (0, 0, 0), (120, 9, 0), (0, 129, 0), (0, 8, 2), (0, 8, -1)):
        ep = moe._CEp(e0, n, acc)
        assert L.moe_forward_ex(good, ctypes.byref(r), ctypes.byref(_packed(max(n, 1), 2048, 768)), None, good,
                                2048, 768, 0, 0, ctypes.byref(ep), good, 1 << 30, None) == -1, (e0, n, acc)
        assert b"expert slice" in L.moe_last_error()
    r.T = 0
    for e0, n, acc in ((0, 128, 0), (120, 8, 1), (0, 1, 1)):
        ep = moe._CEp(e0, n, acc)
        assert L.moe_forward_ex(None, ctypes.byref(r), None, None, None, 2048, 768, 0, 0,
                                ctypes.byref(ep), None, 0, None) == 0
    assert L.moe_forward_ex(None, ctypes.byref(r), None, None, None, 2048, 768, 0, 0,
                            None, None, 0, None) == 0
    r.T = 4
    # router scores + routing: H a positive multiple of 64, k <= E, workspace large enough
    assert L.moe_route_project(None, None, 4, 2048, 128, 8, None, None, None, 0, None) == -1
    assert L.moe_route_project(None, None, 4, 100, 128, 8, None, ctypes.byref(r), None, 0, None) == -2
    assert L.moe_route_project(None, None, 4, 2048, 8, 9, None, ctypes.byref(r), None, 0, None) == -1
    assert L.moe_route_project(None, None, 4, 2048, 128, 8, None, ctypes.byref(r), None, 0, None) == -1
    r.expert_counts = r.route_pos = 4096
    need = L.moe_route_project_workspace_size(4, 2048, 128, 8)
    assert need >= 256 + 4 * 4 * 128
    assert L.moe_route_project(good, good, 4, 2048, 128, 8, good, ctypes.byref(r), good, need - 16,
                               None) == -3
    assert L.moe_route_project(bad, good, 4, 2048, 128, 8, good, ctypes.byref(r), good, need, None) == -1
    assert L.moe_route_project_workspace_size(4, 100, 128, 8) == 0
    # the decode entry: logits required for T > 0, route-direct path only
    assert L.moe_decode_forward(None, good, 4, 128, 8, ctypes.byref(r), ctypes.byref(w), None, good, 2048, 768, 0,
                                0, None, good, 1 << 30, None) == -1
    assert L.moe_decode_forward(good, good, 4, 128, 8, ctypes.byref(r), ctypes.byref(w), None, good, 2048, 768, 0,
                                1, None, good, 1 << 30, None) == -2
    assert L.moe_decode_forward(good, good, 64, 128, 8, ctypes.byref(r), ctypes.byref(w), None, good, 2048, 768, 0,
                                0, None, good, 1 << 30, None) == -2
    # packing rejects in-place, null, and a missing descriptor (whose tag it clears on error)
    d = _packed(4, 256, 64)
    assert L.moe_pack_weights(good, good, 4, 256, 64, 0, good, None, ctypes.byref(d), None) == -1
    assert d.tag == 0
    assert L.moe_pack_weights(good, None, 4, 256, 64, 0, good, good, ctypes.byref(d), None) == -1
    assert L.moe_pack_weights(good, bad, 4, 256, 64, 0, ctypes.c_void_p(8192), ctypes.c_void_p(16384), None,
                              None) == -1


@pytest.mark.skipif(torch.cuda.is_available(),
                    reason="passes fake device addresses; only run where no GPU can be reached")
@pytest.mark.parametrize("field,value", [("E", 64), ("H", 4096), ("I", 512), ("quant", 2), ("tag", 0),
                                         ("tag", 0x12345678)])
def test_packed_descriptor_must_match_the_call(field, value):
    """Weights packed for another shape or format, or a descriptor moe_pack_weights did not
    fill, are rejected with MOE_ERR_INVALID_ARG before anything is enqueued."""
    L = moe.lib()
    good = ctypes.c_void_p(4096)
    r = moe._CRoutes(4096, 4096, 4096, 4096, 4096, 4096, 4, 128, 8)
    w = _packed(128, 2048, 768)
    setattr(w, field, value)
    for path in (0, 1, 2):
        assert L.moe_forward(good, ctypes.byref(r), ctypes.byref(w), None, good, 2048, 768, 0, path, good,
                             1 << 30, None) == -1
        msg = L.moe_last_error()
        assert b"moe_pack_weights" in msg or b"packed for" in msg, msg
    ep = moe._CEp(0, 128, 0)
    assert L.moe_forward_ex(good, ctypes.byref(r), ctypes.byref(w), None, good, 2048, 768, 0, 0, ctypes.byref(ep),
                            good, 1 << 30, None) == -1
    lg = ctypes.c_void_p(4096)
    assert L.moe_decode_forward(lg, good, 4, 128, 8, ctypes.byref(r), ctypes.byref(w), None, good, 2048, 768, 0, 0,
                                None, good, 1 << 30, None) == -1
    # a slice needs weights packed with E = num_experts
    ep = moe._CEp(8, 16, 0)
    assert L.moe_forward_ex(good, ctypes.byref(r), ctypes.byref(_packed(128, 2048, 768)), None, good, 2048, 768, 0,
                            0, ctypes.byref(ep), good, 1 << 30, None) == -1


def test_large_shapes_limits_before_launch():
    """Large T runs on the grouped path (h and y addressed per row tile); what the
    kernels cannot address is rejected on the host with MOE_ERR_UNSUPPORTED."""
    # y = T*k*H*2 bytes well past 2 GiB and 4 GiB: accepted
    assert moe.select_path(70000, 2048, 256, 8, 8) == "grouped"
    assert moe.forward_workspace_size(70000, 2048, 256, 8, 8) > 70000 * 8 * 2048 * 2
    assert moe.select_path(262144, 4096, 1024, 128, 8, "fp8_block128") == "grouped"
    # T*H >= 2^31 and T*k*I >= 2^36 are not
    for args in ((524288, 4096, 512, 128, 8), (1 << 22, 512, 8192, 128, 4)):
        with pytest.raises(moe.MoeError) as ei:
            moe.select_path(*args)
        assert ei.value.code == -2
        assert moe.forward_workspace_size(*args) == 0


def test_workspace_views_layout():
    """The documented inspection views lie inside the workspace and do not overlap."""
    for T, quant, path in ((4096, "fp8_block128", "grouped"), (3, "fp8_block128", "route_direct"),
                           (8, "fp8_per_tensor", "grouped"), (2, "fp8_per_tensor", "route_direct"),
                           (64, "fp8_mx32", "grouped"), (64, "bf16", "grouped")):
        H, I, E, k = 4096, 512, 128, 8
        v = moe.forward_workspace_views(T, H, I, E, k, quant, path)
        n = moe.forward_workspace_size(T, H, I, E, k, quant, path)
        if quant == "bf16":
            assert all(x is None for x in v.values())
            continue
        R = T * k
        sizes = {"x_codes": T * H,
                 "x_scales": {"fp8_per_tensor": 4, "fp8_block128": 4 * T * H // 128, "fp8_mx32": T * H // 32}[quant],
                 "h_codes": R * I if path == "grouped" else 0,
                 "h_scales": {"fp8_per_tensor": 4, "fp8_block128": 4 * R * I // 128, "fp8_mx32": R * I // 32}[quant]}
        spans = []
        for key, size in sizes.items():
            if size == 0:
                assert v[key] is None, (key, quant, path)
                continue
            assert v[key] is not None and v[key] + size <= n, (key, quant, path)
            spans.append((v[key], v[key] + size))
        spans.sort()
        assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:])), (quant, path, spans)


def test_backward_sizes_and_shape_rules():
    """The MX backward's buffer sizes cover what it writes; unsupported shapes give 0."""
    E, H, I = 128, 4096, 512
    w = moe.mx_train_weights_size(E, H, I)
    # five packed operand sets: 3 x (E H 2I) + 2 x (E I H) codes, and their scales (one byte per 32)
    assert w >= (2 + 2 + 1 + 1 + 2) * E * H * I * 33 // 32
    T, k = 4096, 8
    R = T * k
    ws = moe.backward_workspace_size(T, H, I, E, k)
    # g|u, h and dh in fp32, y in bf16, dGU in fp32 and codes, the four transposed operands
    assert ws >= R * (2 * I * 4 + I * 4 + H * 2 + I * 4 + 2 * I * 5) + (2 * H + 3 * I) * (R + 63 * E)
    assert moe.backward_workspace_size(0, H, I, E, k) > 0          # an empty batch still writes dW = 0
    for bad in ((T, 4096 + 64, I, E, k), (T, H, 384, E, k), (T, H, I, 4, 8), (T, 16384, I, E, k)):
        assert moe.backward_workspace_size(*bad) == 0, bad
    assert moe.mx_train_weights_size(E, 4096 + 64, I) == 0
    assert moe.mx_train_weights_size(E, H, 128) == 0


@pytest.mark.skipif(torch.cuda.is_available(),
                    reason="passes fake device addresses; only run where no GPU can be reached")
def test_backward_host_validation_before_any_launch():
    L = moe.lib()
    good = ctypes.c_void_p(4096)
    bad = ctypes.c_void_p(4096 + 8)
    tw = moe._CTrain()
    # preparation: unsupported shape, null pointers, misalignment, short buffer
    assert L.moe_prepare_mx_train_weights(good, good, 4, 320, 256, good, 1 << 40, ctypes.byref(tw), None) == -2
    assert tw.tag == 0
    assert L.moe_prepare_mx_train_weights(None, good, 4, 256, 256, good, 1 << 40, ctypes.byref(tw), None) == -1
    assert L.moe_prepare_mx_train_weights(bad, good, 4, 256, 256, good, 1 << 40, ctypes.byref(tw), None) == -1
    assert L.moe_prepare_mx_train_weights(good, good, 4, 256, 256, good, 16, ctypes.byref(tw), None) == -3
    # backward: descriptor not prepared, E mismatch, misaligned, short workspace
    r = moe._CRoutes()
    r.T, r.E, r.k = 8, 4, 2
    r.topk_ids = r.topk_weights = r.expert_offsets = r.perm = r.route_pos = 4096
    w = moe._CTrain(4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096, 4, 256, 256, 0, moe._CPacked(), moe._CScales())
    args = [good, ctypes.byref(r), ctypes.byref(w), good, good, good, good, good, good, 1 << 40, None]
    assert L.moe_backward(*args) == -1 and b"moe_prepare_mx_train_weights" in L.moe_last_error()
    w.tag = moe.TRAIN_TAG
    w.E = 8
    assert L.moe_backward(*args) == -1
    w.E = 4
    args[3] = bad
    assert L.moe_backward(*args) == -1
    args[3] = good
    args[9] = 16
    assert L.moe_backward(*args) == -3
    w.H = 320
    assert L.moe_backward(*args) == -2
    # the route backward: null routes, k > E, an empty batch, misalignment
    assert L.moe_route_backward(None, good, good, None) == -1
    r2 = moe._CRoutes()
    r2.T, r2.E, r2.k = 4, 4, 8
    assert L.moe_route_backward(ctypes.byref(r2), good, good, None) == -1
    r2.T, r2.E, r2.k = 0, 8, 2
    assert L.moe_route_backward(ctypes.byref(r2), None, None, None) == 0
    r2.T = 4
    r2.topk_ids = r2.topk_weights = 4096
    assert L.moe_route_backward(ctypes.byref(r2), bad, good, None) == -1
    assert L.moe_route_backward(ctypes.byref(r2), good, None, None) == -1


def test_launch_info_shape():
    li = moe.forward_launch_info(8192, 2048, 768, 128, 8)
    assert li["path"] == "grouped" and li["gate_up_split"] == 0
    li = moe.forward_launch_info(1, 2048, 768, 128, 8, "fp8_block128", "route_direct")
    assert li["path"] == "route_direct" and li["gate_up_split"] in (1, 2, 4) and li["gate_up_waves"] >= 1
    assert li["down_form"] in (0, 1) and li["down_parts"] in (1, 2, 4)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it exits with status 2 and a message,
    before touching torch or the device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
