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
    # MX FP8 runs on the grouped path only, H and I multiples of 256
    assert moe.select_path(1, 2048, 768, 128, 8, "fp8_mx32") == "grouped"
    with pytest.raises(moe.MoeError):
        moe.select_path(1, 2048, 768, 128, 8, "fp8_mx32", "route_direct")
    with pytest.raises(moe.MoeError):
        moe.select_path(64, 2048, 192, 128, 8, "fp8_mx32")
    assert moe.select_path(64, 2048, 768, 128, 8, "bf16", "route_direct") == "route_direct"


@pytest.mark.parametrize("args,code", [
    ((1, 2048, 768, 4, 8, "bf16", "auto"), -1),      # k > E
    ((1, 2048, 768, 600, 8, "bf16", "auto"), -1),    # E > 512
    ((1, 2000, 768, 128, 8, "bf16", "auto"), -2),    # H % 128
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


@pytest.mark.skipif(torch.cuda.is_available(),
                    reason="passes fake device addresses; only run where no GPU can be reached")
def test_host_validation_before_any_launch():
    L = moe.lib()
    r = moe._CRoutes()
    # k > E is rejected on the host (no device pointer is touched)
    assert L.moe_route(None, 4, 4, 8, ctypes.byref(r), None, 0, None) == -1
    assert L.moe_route(None, 4, 8, 2, None, None, 0, None) == -1
    # null routes / null pointers / bad quant
    assert L.moe_forward(None, None, None, None, None, None, 2048, 768, 0, 0, None, 0, None) == -1
    r.T, r.E, r.k = 4, 128, 8
    assert L.moe_forward(None, ctypes.byref(r), None, None, None, None, 2048, 768, 0, 0, None, 0,
                         None) == -1
    assert L.moe_forward(None, ctypes.byref(r), None, None, None, None, 2048, 768, 7, 0, None, 0,
                         None) == -1
    # T = 0 is a valid empty call: nothing to do, no launch
    r.T = 0
    assert L.moe_forward(None, ctypes.byref(r), None, None, None, None, 2048, 768, 0, 0, None, 0,
                         None) == 0
    # misaligned pointers are rejected
    r.T = 4
    r.topk_ids = r.topk_weights = r.expert_offsets = r.perm = 4096
    bad = ctypes.c_void_p(4096 + 8)
    good = ctypes.c_void_p(4096)
    assert L.moe_forward(bad, ctypes.byref(r), good, good, None, good, 2048, 768, 0, 0, good, 1 << 30,
                         None) == -1
    # short workspace
    assert L.moe_forward(good, ctypes.byref(r), good, good, None, good, 2048, 768, 0, 0, good, 16,
                         None) == -3
    # fp8 needs scales
    assert L.moe_forward(good, ctypes.byref(r), good, good, None, good, 2048, 768, 1, 0, good, 1 << 30,
                         None) == -1
    # expert slices: [expert_begin, expert_begin + num_experts) inside [0, E), accumulate 0 or 1
    for e0, n, acc in ((-1, 4, 0), (0, 0, 0), (120, 9, 0), (0, 129, 0), (0, 8, 2), (0, 8, -1)):
        ep = moe._CEp(e0, n, acc)
        assert L.moe_forward_ex(good, ctypes.byref(r), good, good, None, good, 2048, 768, 0, 0,
                                ctypes.byref(ep), good, 1 << 30, None) == -1, (e0, n, acc)
        assert b"expert slice" in L.moe_last_error()
    r.T = 0
    for e0, n, acc in ((0, 128, 0), (120, 8, 1), (0, 1, 1)):
        ep = moe._CEp(e0, n, acc)
        assert L.moe_forward_ex(None, ctypes.byref(r), None, None, None, None, 2048, 768, 0, 0,
                                ctypes.byref(ep), None, 0, None) == 0
    assert L.moe_forward_ex(None, ctypes.byref(r), None, None, None, None, 2048, 768, 0, 0,
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
    assert L.moe_decode_forward(None, good, 4, 128, 8, ctypes.byref(r), good, good, None, good, 2048, 768, 0, 0,
                                None, good, 1 << 30, None) == -1
    assert L.moe_decode_forward(good, good, 4, 128, 8, ctypes.byref(r), good, good, None, good, 2048, 768, 0, 1,
                                None, good, 1 << 30, None) == -2
    assert L.moe_decode_forward(good, good, 64, 128, 8, ctypes.byref(r), good, good, None, good, 2048, 768, 0, 0,
                                None, good, 1 << 30, None) == -2
    # packing rejects in-place and null
    assert L.moe_pack_weights(good, good, 4, 256, 64, 0, good, None, None) == -1
    assert L.moe_pack_weights(good, None, 4, 256, 64, 0, good, good, None) == -1


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it exits with status 2 and a message,
    before touching torch or the device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
