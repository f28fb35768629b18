"""MI355X (gfx950) MoE FFN forward: Python binding of the C ABI in include/moe.h.

This module only marshals arguments: torch supplies device memory and the
stream, and every step of the layer runs in the HIP kernels of
``libmoe_mi355x.so``.  There is no fallback: if the library is not built, or
no GPU is present, the calls raise.

    routes = route(logits, k)                         # top-k + grouping by expert
    w = pack_weights(w_gate_up, w_down, quant)        # once per weight set
    out = forward(x, routes, w, scales=(s_gu, s_d), path="auto")

    tw = prepare_mx_train_weights(w_gate_up_bf16, w_down_bf16)   # per weight update
    g = backward(x, routes, tw, dout)                 # dx, dgate, dw_gate_up, dw_down
"""
from __future__ import annotations

import ctypes
import os

import torch

_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_DIR, "libmoe_mi355x.so")

QUANT = {"bf16": 0, "fp8_per_tensor": 1, "fp8_block128": 2, "fp8_mx32": 3}
PATH = {"auto": 0, "grouped": 1, "route_direct": 2}
PATH_NAME = {v: k for k, v in PATH.items()}
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED",
          -3: "MOE_ERR_WORKSPACE", -4: "MOE_ERR_HIP"}

EXPORTED = ["moe_route_workspace_size", "moe_route", "moe_route_project_workspace_size",
            "moe_route_project", "moe_pack_weights", "moe_pack_mx_scales", "moe_select_path",
            "moe_forward_workspace_size", "moe_forward_workspace_views", "moe_forward_launch_info",
            "moe_forward", "moe_forward_ex", "moe_decode_forward", "moe_decode_forward_noalloc",
            "moe_forward_profiled", "moe_forward_timed",
            "moe_mx_train_weights_size", "moe_prepare_mx_train_weights", "moe_backward_workspace_size",
            "moe_backward", "moe_backward_profiled", "moe_route_backward",
            "moe_last_error"]
PACKED_TAG = 0x4D6F4557
TRAIN_TAG = 0x4D6F4542


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class _CRoutes(ctypes.Structure):
    _fields_ = [("topk_ids", ctypes.c_void_p), ("topk_weights", ctypes.c_void_p),
                ("expert_counts", ctypes.c_void_p), ("expert_offsets", ctypes.c_void_p),
                ("perm", ctypes.c_void_p), ("route_pos", ctypes.c_void_p),
                ("T", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32)]


class _CScales(ctypes.Structure):
    _fields_ = [("w_gate_up_scale", ctypes.c_void_p), ("w_down_scale", ctypes.c_void_p)]


class _CEp(ctypes.Structure):
    _fields_ = [("expert_begin", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("accumulate", ctypes.c_int32)]


class _CPacked(ctypes.Structure):
    _fields_ = [("gate_up", ctypes.c_void_p), ("down", ctypes.c_void_p), ("E", ctypes.c_int32),
                ("H", ctypes.c_int32), ("I", ctypes.c_int32), ("quant", ctypes.c_int32),
                ("tag", ctypes.c_uint32)]


class _CTrain(ctypes.Structure):
    _fields_ = [("gate_up_k", ctypes.c_void_p), ("gate_up_k_scales", ctypes.c_void_p),
                ("down_k", ctypes.c_void_p), ("down_k_scales", ctypes.c_void_p),
                ("down_t", ctypes.c_void_p), ("down_t_scales", ctypes.c_void_p),
                ("gate_up_t", ctypes.c_void_p), ("gate_up_t_scales", ctypes.c_void_p),
                ("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32), ("tag", ctypes.c_uint32),
                ("forward", _CPacked), ("forward_scales", _CScales)]


class _CViews(ctypes.Structure):
    _fields_ = [("x_codes", ctypes.c_int64), ("x_scales", ctypes.c_int64), ("h_codes", ctypes.c_int64),
                ("h_scales", ctypes.c_int64)]


class _CLaunch(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("gate_up_split", ctypes.c_int32), ("gate_up_waves", ctypes.c_int32),
                ("down_form", ctypes.c_int32), ("down_parts", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.moe_route_workspace_size.restype = sz
    L.moe_route_workspace_size.argtypes = [i32, i32, i32]
    L.moe_route.restype = i32
    L.moe_route.argtypes = [P, i32, i32, i32, ctypes.POINTER(_CRoutes), P, sz, P]
    L.moe_pack_weights.restype = i32
    L.moe_route_project_workspace_size.restype = sz
    L.moe_route_project_workspace_size.argtypes = [i32, i32, i32, i32]
    L.moe_route_project.restype = i32
    L.moe_route_project.argtypes = [P, P, i32, i32, i32, i32, P, ctypes.POINTER(_CRoutes), P, sz, P]
    L.moe_pack_mx_scales.restype = i32
    L.moe_pack_mx_scales.argtypes = [P, P, i32, i32, i32, P, P, P]
    L.moe_pack_weights.argtypes = [P, P, i32, i32, i32, i32, P, P, ctypes.POINTER(_CPacked), P]
    L.moe_forward_workspace_views.restype = i32
    L.moe_forward_workspace_views.argtypes = [i32] * 7 + [ctypes.POINTER(_CViews)]
    L.moe_forward_launch_info.restype = i32
    L.moe_forward_launch_info.argtypes = [i32] * 7 + [ctypes.POINTER(_CLaunch)]
    L.moe_select_path.restype = i32
    L.moe_select_path.argtypes = [i32] * 7
    L.moe_forward_workspace_size.restype = sz
    L.moe_forward_workspace_size.argtypes = [i32] * 7
    L.moe_forward.restype = i32
    L.moe_forward.argtypes = [P, ctypes.POINTER(_CRoutes), ctypes.POINTER(_CPacked), ctypes.POINTER(_CScales), P,
                              i32, i32, i32, i32, P, sz, P]
    L.moe_forward_ex.restype = i32
    L.moe_forward_ex.argtypes = L.moe_forward.argtypes[:9] + [ctypes.POINTER(_CEp)] + \
        L.moe_forward.argtypes[9:]
    L.moe_decode_forward.restype = i32
    L.moe_decode_forward.argtypes = [P, P, i32, i32, i32, ctypes.POINTER(_CRoutes), ctypes.POINTER(_CPacked),
                                     ctypes.POINTER(_CScales), P, i32, i32, i32, i32, ctypes.POINTER(_CEp), P, sz, P]
    L.moe_decode_forward_noalloc.restype = i32
    L.moe_decode_forward_noalloc.argtypes = L.moe_decode_forward.argtypes[:14] + [P]
    L.moe_forward_timed.restype = i32
    L.moe_forward_timed.argtypes = L.moe_forward.argtypes + [P, P]
    L.moe_forward_profiled.restype = i32
    L.moe_forward_profiled.argtypes = L.moe_forward.argtypes + [ctypes.POINTER(ctypes.c_void_p), i32,
                                                               ctypes.POINTER(ctypes.c_int),
                                                               ctypes.POINTER(ctypes.c_char_p)]
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_mx_train_weights_size.restype = sz
    L.moe_mx_train_weights_size.argtypes = [i32, i32, i32]
    L.moe_prepare_mx_train_weights.argtypes = [P, P, i32, i32, i32, P, sz, ctypes.POINTER(_CTrain), P]
    L.moe_backward_workspace_size.restype = sz
    L.moe_backward_workspace_size.argtypes = [i32] * 5
    L.moe_backward.argtypes = [P, ctypes.POINTER(_CRoutes), ctypes.POINTER(_CTrain), P, P, P, P, P, P, sz, P]
    L.moe_backward_profiled.argtypes = L.moe_backward.argtypes + [ctypes.POINTER(ctypes.c_void_p), i32,
                                                                  ctypes.POINTER(ctypes.c_int),
                                                                  ctypes.POINTER(ctypes.c_char_p)]
    L.moe_route_backward.argtypes = [ctypes.POINTER(_CRoutes), P, P, P]
    L.moe_last_error.argtypes = []
    _lib = L
    return L


def _check(rc: int):
    if rc != 0:
        raise MoeError(rc, lib().moe_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _need_cuda(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class Routes:
    """Device routing arrays of T tokens over E experts (see moe_routes in moe.h)."""

    def __init__(self, T: int, E: int, k: int, device):
        i32 = dict(dtype=torch.int32, device=device)
        self.T, self.E, self.k = T, E, k
        self.topk_ids = torch.empty((T, k), **i32)
        self.topk_weights = torch.empty((T, k), dtype=torch.float32, device=device)
        self.expert_counts = torch.empty(E, **i32)
        self.expert_offsets = torch.empty(E + 1, **i32)
        self.perm = torch.empty(T * k, **i32)
        self.route_pos = torch.empty(T * k, **i32)

    def c_struct(self) -> _CRoutes:
        return _CRoutes(self.topk_ids.data_ptr(), self.topk_weights.data_ptr(),
                        self.expert_counts.data_ptr(), self.expert_offsets.data_ptr(),
                        self.perm.data_ptr(), self.route_pos.data_ptr(), self.T, self.E, self.k)


def route_workspace_size(T: int, E: int, k: int) -> int:
    return int(lib().moe_route_workspace_size(T, E, k))


def route(logits: torch.Tensor, k: int, out: Routes | None = None,
          workspace: torch.Tensor | None = None, stream=None) -> Routes:
    """Top-k routing of fp32 logits [T, E] and its grouped form (moe_route)."""
    _need_cuda(logits, "logits")
    if logits.dtype != torch.float32 or logits.dim() != 2:
        raise ValueError("logits must be float32 [T, E]")
    T, E = logits.shape
    out = out if out is not None else Routes(T, E, k, logits.device)
    need = route_workspace_size(T, E, k)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    cs = out.c_struct()
    _check(lib().moe_route(_ptr(logits), T, E, k, ctypes.byref(cs), _ptr(workspace),
                           0 if workspace is None else workspace.numel(),
                           _stream(logits.device, stream)))
    return out


def route_project_workspace_size(T: int, H: int, E: int, k: int) -> int:
    return int(lib().moe_route_project_workspace_size(T, H, E, k))


def route_project(x: torch.Tensor, w_router: torch.Tensor, k: int, out: Routes | None = None,
                  logits: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """Router scores x W_r and the routing from them (moe_route_project).

    x bf16 [T, H], w_router fp32 [H, E]; returns (Routes, logits fp32 [T, E]).
    A workspace passed in must have been zero-filled before its first use (the
    call leaves its arrival counter at zero)."""
    _need_cuda(x, "x")
    _need_cuda(w_router, "w_router")
    if x.element_size() != 2 or x.dim() != 2:
        raise ValueError("x must be a bf16 [T, H] tensor")
    if w_router.dtype != torch.float32 or w_router.dim() != 2 or w_router.shape[0] != x.shape[1]:
        raise ValueError("w_router must be float32 [H, E]")
    T, H = x.shape
    E = w_router.shape[1]
    out = out if out is not None else Routes(T, E, k, x.device)
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    need = route_project_workspace_size(T, H, E, k)
    if workspace is None and need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=x.device)
    cs = out.c_struct()
    _check(lib().moe_route_project(_ptr(x), _ptr(w_router), T, H, E, k, _ptr(logits), ctypes.byref(cs),
                                   _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                   _stream(x.device, stream)))
    return out, logits


class PackedWeights:
    """Expert weights re-laid by moe_pack_weights: the two packed device
    buffers and the C descriptor (shape, format, tag) the forward calls check."""

    def __init__(self, gate_up: torch.Tensor, down: torch.Tensor, desc: _CPacked):
        self.gate_up, self.down, self.desc = gate_up, down, desc

    E = property(lambda self: self.desc.E)
    H = property(lambda self: self.desc.H)
    I = property(lambda self: self.desc.I)
    quant = property(lambda self: {v: k for k, v in QUANT.items()}[self.desc.quant])


def pack_weights(w_gate_up: torch.Tensor, w_down: torch.Tensor, quant: str = "bf16", stream=None) -> PackedWeights:
    """Re-lay [E,H,2I] and [E,I,H] weights into the packed K-contiguous form (moe_pack_weights)."""
    _need_cuda(w_gate_up, "w_gate_up")
    _need_cuda(w_down, "w_down")
    E, H, I2 = w_gate_up.shape
    I = I2 // 2
    if tuple(w_down.shape) != (E, I, H):
        raise ValueError("w_down must be [E, I, H]")
    pgu = torch.empty_like(w_gate_up)
    pd = torch.empty_like(w_down)
    desc = _CPacked()
    _check(lib().moe_pack_weights(_ptr(w_gate_up), _ptr(w_down), E, H, I, QUANT[quant], _ptr(pgu),
                                  _ptr(pd), ctypes.byref(desc), _stream(w_gate_up.device, stream)))
    return PackedWeights(pgu, pd, desc)


def _need_packed(w):
    if not isinstance(w, PackedWeights):
        raise TypeError("weights must be the PackedWeights that pack_weights returned")
    return w


def pack_mx_scales(s_gate_up: torch.Tensor, s_down: torch.Tensor, stream=None):
    """Re-lay MX E8M0 scale bytes [E,H/32,2I] and [E,I/32,H] into the order the MX
    GEMM reads them (moe_pack_mx_scales); pass the result as `scales`."""
    _need_cuda(s_gate_up, "s_gate_up")
    _need_cuda(s_down, "s_down")
    if s_gate_up.dtype != torch.uint8 or s_down.dtype != torch.uint8:
        raise ValueError("MX scales are uint8 E8M0 bytes")
    E, H32, I2 = s_gate_up.shape
    H, I = H32 * 32, I2 // 2
    if tuple(s_down.shape) != (E, I // 32, H):
        raise ValueError("s_down must be [E, I/32, H]")
    pgu = torch.empty_like(s_gate_up)
    pd = torch.empty_like(s_down)
    _check(lib().moe_pack_mx_scales(_ptr(s_gate_up), _ptr(s_down), E, H, I, _ptr(pgu), _ptr(pd),
                                    _stream(s_gate_up.device, stream)))
    return pgu, pd


def select_path(T, H, I, E, k, quant="bf16", path="auto") -> str:
    rc = lib().moe_select_path(T, H, I, E, k, QUANT[quant], PATH[path])
    _check(rc if rc < 0 else 0)
    return PATH_NAME[rc]


def forward_workspace_size(T, H, I, E, k, quant="bf16", path="auto") -> int:
    return int(lib().moe_forward_workspace_size(T, H, I, E, k, QUANT[quant], PATH[path]))


def forward_workspace_views(T, H, I, E, k, quant="bf16", path="auto") -> dict:
    """Byte offsets into the forward workspace of the quantised x and h codes and
    scales a call leaves there (moe_forward_workspace_views); None where absent."""
    v = _CViews()
    _check(lib().moe_forward_workspace_views(T, H, I, E, k, QUANT[quant], PATH[path], ctypes.byref(v)))
    return {f: (None if getattr(v, f) < 0 else int(getattr(v, f))) for f, _ in _CViews._fields_}


def forward_launch_info(T, H, I, E, k, quant="bf16", path="auto") -> dict:
    """The launch shape a forward call with these arguments takes (moe_forward_launch_info)."""
    li = _CLaunch()
    _check(lib().moe_forward_launch_info(T, H, I, E, k, QUANT[quant], PATH[path], ctypes.byref(li)))
    d = {f: int(getattr(li, f)) for f, _ in _CLaunch._fields_}
    d["path"] = PATH_NAME[d["path"]]
    return d


def decode_forward(logits: torch.Tensor, x: torch.Tensor, k: int, weights: PackedWeights,
                   quant: str | None = None, scales=None, out: torch.Tensor | None = None,
                   routes: Routes | None = None, path: str = "auto", workspace: torch.Tensor | None = None,
                   stream=None, expert_begin: int = 0, num_experts: int | None = None, accumulate: bool = False):
    """Routing and the route-direct layer in one call (moe_decode_forward): returns
    (out, routes); routes carries topk_ids and topk_weights (counts, offsets,
    perm and route_pos are not written)."""
    _need_cuda(logits, "logits")
    _need_cuda(x, "x")
    if logits.dtype != torch.float32 or logits.dim() != 2:
        raise ValueError("logits must be float32 [T, E]")
    T, E = logits.shape
    if x.element_size() != 2 or x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x must be a bf16 [T, H] tensor with the logits' T")
    H = x.shape[1]
    w = _need_packed(weights)
    quant = w.quant if quant is None else quant
    I = w.I
    if accumulate and out is None:
        raise ValueError("accumulate needs the output to add into")
    routes = routes if routes is not None else Routes(T, E, k, x.device)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    need = forward_workspace_size(T, H, I, E, k, quant, path)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    cs = routes.c_struct()
    sc = _CScales(None, None) if scales is None else _CScales(scales[0].data_ptr(), scales[1].data_ptr())
    ep = _CEp(expert_begin, E - expert_begin if num_experts is None else num_experts, int(bool(accumulate)))
    _check(lib().moe_decode_forward(_ptr(logits), _ptr(x), T, E, k, ctypes.byref(cs), ctypes.byref(w.desc),
                                    ctypes.byref(sc), _ptr(out), H, I, QUANT[quant], PATH[path],
                                    ctypes.byref(ep), _ptr(workspace), workspace.numel(), _stream(x.device, stream)))
    return out, routes


def decode_forward_noalloc(logits: torch.Tensor, x: torch.Tensor, k: int, weights: PackedWeights,
                           out: torch.Tensor, routes: Routes, quant: str | None = None, scales=None,
                           path: str = "auto", stream=None, expert_begin: int = 0, num_experts: int | None = None,
                           accumulate: bool = False):
    """decode_forward with the library's own static workspace (moe_decode_forward_noalloc):
    the caller passes preallocated `out` and `routes`; the call allocates nothing."""
    _need_cuda(logits, "logits")
    _need_cuda(x, "x")
    _need_cuda(out, "out")
    T, E = logits.shape
    H = x.shape[1]
    w = _need_packed(weights)
    quant = w.quant if quant is None else quant
    cs = routes.c_struct()
    sc = _CScales(None, None) if scales is None else _CScales(scales[0].data_ptr(), scales[1].data_ptr())
    ep = _CEp(expert_begin, E - expert_begin if num_experts is None else num_experts, int(bool(accumulate)))
    _check(lib().moe_decode_forward_noalloc(_ptr(logits), _ptr(x), T, E, k, ctypes.byref(cs), ctypes.byref(w.desc),
                                            ctypes.byref(sc), _ptr(out), H, w.I, QUANT[quant], PATH[path],
                                            ctypes.byref(ep), _stream(x.device, stream)))
    return out


def forward(x: torch.Tensor, routes: Routes, weights: PackedWeights,
            quant: str | None = None, scales=None, out: torch.Tensor | None = None, path: str = "auto",
            workspace: torch.Tensor | None = None, stream=None, events=None,
            expert_begin: int = 0, num_experts: int | None = None, accumulate: bool = False,
            device_events=None):
    """Layer output bf16 [T, H] (moe_forward).

    weights: what pack_weights returned; quant defaults to the format they were
    packed for (a different quant is passed through and rejected by the library).
    expert_begin / num_experts / accumulate select an expert slice and a
    shared output (moe_forward_ex): the packed weights and scales then hold
    experts [expert_begin, expert_begin + num_experts) only, the routes stay
    global, and accumulate=True adds the slice's sum into `out`.

    With events (a list of torch.cuda.Event(enable_timing=True) or None) it
    calls moe_forward_profiled instead, which attaches events[0] to the first
    kernel's start and events[i] to the end of stage i's last kernel (None
    entries take no event; no marker packet between kernels), and returns
    (out, stage_names).

    With device_events=(start, end) (torch.cuda.Event(enable_timing=True)) it
    calls moe_forward_timed: start/end are attached to the first and last kernel
    dispatches, so start.elapsed_time(end) is the forward's device span."""
    _need_cuda(x, "x")
    if x.element_size() != 2 or x.dim() != 2:
        raise ValueError("x must be a bf16 [T, H] tensor")
    T, H = x.shape
    w = _need_packed(weights)
    quant = w.quant if quant is None else quant
    I = w.I
    if routes.T != T:
        raise ValueError("routes and x disagree on T")
    ep = None
    if expert_begin != 0 or num_experts is not None or accumulate:
        if events is not None:
            raise ValueError("stage events are not recorded for an expert slice")
        if accumulate and out is None:
            raise ValueError("accumulate needs the output to add into")
        ep = _CEp(expert_begin, routes.E - expert_begin if num_experts is None else num_experts,
                  int(bool(accumulate)))
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    need = forward_workspace_size(T, H, I, routes.E, routes.k, quant, path)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    cs = routes.c_struct()
    sc = _CScales(None, None)
    if scales is not None:
        sc = _CScales(scales[0].data_ptr(), scales[1].data_ptr())
    args = (_ptr(x), ctypes.byref(cs), ctypes.byref(w.desc), ctypes.byref(sc),
            _ptr(out), H, I, QUANT[quant], PATH[path], _ptr(workspace), workspace.numel(),
            _stream(x.device, stream))
    if ep is not None:
        _check(lib().moe_forward_ex(*args[:9], ctypes.byref(ep), *args[9:]))
        return out
    if device_events is not None:
        st = stream if stream is not None else torch.cuda.current_stream(x.device)
        for ev in device_events:
            if not ev.cuda_event:
                ev.record(st)       # torch creates the underlying event on first record
        _check(lib().moe_forward_timed(*args, ctypes.c_void_p(device_events[0].cuda_event),
                                       ctypes.c_void_p(device_events[1].cuda_event)))
        return out
    if events is None:
        _check(lib().moe_forward(*args))
        return out
    st = stream if stream is not None else torch.cuda.current_stream(x.device)
    for ev in events:
        if ev is not None and not ev.cuda_event:
            ev.record(st)           # torch creates the underlying event on first record
    handles = (ctypes.c_void_p * len(events))(*[ev.cuda_event if ev is not None else None for ev in events])
    n = ctypes.c_int(0)
    names = ctypes.c_char_p()
    _check(lib().moe_forward_profiled(*args, handles, len(events), ctypes.byref(n), ctypes.byref(names)))
    return out, names.value.decode().split(",")[: n.value]


class TrainWeights:
    """The packed MX operand sets moe_prepare_mx_train_weights builds from bf16
    master weights (one device buffer) and their C descriptor.  `forward` and
    `forward_scales` are the MX forward's weights and scales, for forward()
    with quant "fp8_mx32"."""

    def __init__(self, buf: torch.Tensor, desc: _CTrain):
        self.buf, self.desc = buf, desc
        E, H, I = desc.E, desc.H, desc.I
        base = buf.data_ptr()

        def view(ptr, n):
            return buf[ptr - base:ptr - base + n]

        f = desc.forward
        self.forward = PackedWeights(view(f.gate_up, 2 * E * H * I), view(f.down, E * H * I), f)
        self.forward_scales = (view(desc.forward_scales.w_gate_up_scale, 2 * E * H * I // 32),
                               view(desc.forward_scales.w_down_scale, E * H * I // 32))

    E = property(lambda self: self.desc.E)
    H = property(lambda self: self.desc.H)
    I = property(lambda self: self.desc.I)


def mx_train_weights_size(E: int, H: int, I: int) -> int:
    return int(lib().moe_mx_train_weights_size(E, H, I))


def prepare_mx_train_weights(w_gate_up: torch.Tensor, w_down: torch.Tensor, stream=None) -> TrainWeights:
    """bf16 master weights [E,H,2I], [E,I,H] -> the MX operand sets of the
    recomputed forward and of the input gradients (moe_prepare_mx_train_weights)."""
    _need_cuda(w_gate_up, "w_gate_up")
    _need_cuda(w_down, "w_down")
    if w_gate_up.element_size() != 2 or w_down.element_size() != 2:
        raise ValueError("master weights must be bf16")
    E, H, I2 = w_gate_up.shape
    I = I2 // 2
    if tuple(w_down.shape) != (E, I, H):
        raise ValueError("w_down must be [E, I, H]")
    need = mx_train_weights_size(E, H, I)
    buf = torch.empty(max(need, 256), dtype=torch.uint8, device=w_gate_up.device)
    desc = _CTrain()
    _check(lib().moe_prepare_mx_train_weights(_ptr(w_gate_up), _ptr(w_down), E, H, I, _ptr(buf), need,
                                              ctypes.byref(desc), _stream(w_gate_up.device, stream)))
    return TrainWeights(buf, desc)


def backward_workspace_size(T: int, H: int, I: int, E: int, k: int) -> int:
    return int(lib().moe_backward_workspace_size(T, H, I, E, k))


def backward(x: torch.Tensor, routes: Routes, weights: TrainWeights, dout: torch.Tensor,
             workspace: torch.Tensor | None = None, stream=None, events=None, out=None):
    """The layer's gradients for the upstream gradient dout bf16 [T, H]
    (moe_backward): dict(dx bf16 [T,H], dgate fp32 [T,k], dw_gate_up bf16
    [E,H,2I], dw_down bf16 [E,I,H]).  With events (torch.cuda.Event list) it
    calls moe_backward_profiled and also returns the stage names."""
    _need_cuda(x, "x")
    _need_cuda(dout, "dout")
    if not isinstance(weights, TrainWeights):
        raise TypeError("weights must be what prepare_mx_train_weights returned")
    T, H = x.shape
    E, k, I = routes.E, routes.k, weights.I
    dev = x.device
    if out is None:
        out = {"dx": torch.empty((T, H), dtype=torch.bfloat16, device=dev),
               "dgate": torch.empty((T, k), dtype=torch.float32, device=dev),
               "dw_gate_up": torch.empty((E, H, 2 * I), dtype=torch.bfloat16, device=dev),
               "dw_down": torch.empty((E, I, H), dtype=torch.bfloat16, device=dev)}
    need = backward_workspace_size(T, H, I, E, k)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    cs = routes.c_struct()
    args = (_ptr(x), ctypes.byref(cs), ctypes.byref(weights.desc), _ptr(dout), _ptr(out["dx"]),
            _ptr(out["dgate"]), _ptr(out["dw_gate_up"]), _ptr(out["dw_down"]), _ptr(workspace),
            workspace.numel(), _stream(dev, stream))
    if events is None:
        _check(lib().moe_backward(*args))
        return out
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    for ev in events:
        if ev is not None and not ev.cuda_event:
            ev.record(st)
    handles = (ctypes.c_void_p * len(events))(*[ev.cuda_event if ev is not None else None for ev in events])
    n = ctypes.c_int(0)
    names = ctypes.c_char_p()
    _check(lib().moe_backward_profiled(*args, handles, len(events), ctypes.byref(n), ctypes.byref(names)))
    return out, names.value.decode().split(",")[: n.value]


def route_backward(routes: Routes, dgate: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """The gates' gradient dgate fp32 [T, k] taken to the router logits: fp32 [T, E]
    (moe_route_backward)."""
    _need_cuda(dgate, "dgate")
    if dgate.dtype != torch.float32 or tuple(dgate.shape) != (routes.T, routes.k):
        raise ValueError("dgate must be float32 [T, k]")
    if out is None:
        out = torch.empty((routes.T, routes.E), dtype=torch.float32, device=dgate.device)
    cs = routes.c_struct()
    _check(lib().moe_route_backward(ctypes.byref(cs), _ptr(dgate), _ptr(out), _stream(dgate.device, stream)))
    return out
