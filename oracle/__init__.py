"""CPU oracle of the MoE FFN forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU product path neither imports nor
calls it.  The arithmetic lives in ``moe_oracle.c`` (plain C, fp64
accumulation); this module only marshals numpy arrays through ctypes.

Functions and what they follow (page titles and sections):
  router_logits -- the per-expert router scores of a token, a bias-free linear
                map x W_r ("Port necessary FBGEMM MoE kernels", Benchmarks: the
                MoE module of 16 experts, top 8; the router's form is not
                printed, the linear map is the plain reading).
  route      -- token-choice top-k routing and its grouped form: per-expert
                counts, exclusive prefix, stable route permutation and its
                inverse ("Port necessary FBGEMM MoE kernels", Summary: index
                shuffling; "perf: add small-batch route MMA for MoE",
                Motivation: count/sort, prefix).
  forward    -- the layer output for a list of tokens: Gate/Up projection,
                SwiGLU, optional FP8 requantisation, Down projection, top-k
                weighted combine ("perf: add small-batch route MMA for MoE",
                Summary and Motivation; "Port necessary FBGEMM MoE kernels",
                Summary: scatter_add_dense_tokens).
  gate_up_h  -- the SwiGLU output of listed routes (the tensor the Down-input
                quantisation scales are taken over; same passages as forward).
  quantise_activations, e4m3_encode/decode, bf16_decode -- the FP8 per-tensor
                and 128-channel blockwise activation quantisation and the
                codecs ("perf: add small-batch route MMA for MoE", Summary).
  backward_mx -- the layer's gradients (input, gates, both expert weights)
                for an upstream gradient under the MX training recipe: every
                backward product on MX operands quantised along its own
                reduction dimension, the weight gradients' operands along each
                expert's routes ("[mxfp8 moe training] add per group blocked
                scale kernels", Summary and stacked pull requests: the dim1
                cast in the backward, per-group padded scale rows); exact=True
                is the same calculus with no quantiser.
  route_backward -- the gates' gradient taken to the logits: the softmax
                Jacobian over the k picks (the picks are piecewise constant).
  mx_scale_byte, quantise_group_mx, quant "fp8_mx32" -- MX FP8: e4m3 codes
                with one power-of-two (E8M0) scale per 32 values along K
                ("[mxfp8 moe training] add per group blocked scale kernels",
                Summary: mxfp8 scales; the OCP MX scale rule).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None

QUANT = {"bf16": 0, "fp8_per_tensor": 1, "fp8_block128": 2, "fp8_mx32": 3}


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build_oracle
        build_oracle.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int
    lib.oracle_num_threads.restype = i32
    lib.oracle_bf16_decode.restype = ctypes.c_float
    lib.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_scale_from_amax.restype = ctypes.c_float
    lib.oracle_scale_from_amax.argtypes = [ctypes.c_float]
    lib.oracle_mx_scale_byte.restype = ctypes.c_uint8
    lib.oracle_mx_scale_byte.argtypes = [ctypes.c_float]
    lib.oracle_quantise_group_mx.restype = ctypes.c_uint8
    lib.oracle_quantise_group_mx.argtypes = [P, ctypes.c_long, P]
    lib.oracle_quantise_group.restype = ctypes.c_float
    lib.oracle_quantise_group.argtypes = [P, ctypes.c_long, P]
    lib.oracle_router_logits.restype = None
    lib.oracle_router_logits.argtypes = [P, P, i32, i32, i32, P]
    lib.oracle_route.restype = None
    lib.oracle_route.argtypes = [P, i32, i32, i32, P, P, P, P, P, P]
    lib.oracle_forward.restype = i32
    lib.oracle_forward.argtypes = [P, i32, i32, i32, i32, i32, P, P, P, P, P, P,
                                   i32, P, i32, P]
    lib.oracle_forward_ep.restype = i32
    lib.oracle_forward_ep.argtypes = [P, i32, i32, i32, i32, i32, P, P, P, P, P, P,
                                      i32, i32, i32, P, i32, P]
    lib.oracle_quantise_activations.restype = i32
    lib.oracle_quantise_activations.argtypes = [P, i32, i32, i32, P, P]
    lib.oracle_gate_up_h.restype = i32
    lib.oracle_gate_up_h.argtypes = [P, i32, i32, i32, i32, i32, P, P, P, i32, P, ctypes.c_long, P]
    lib.oracle_route_backward.restype = i32
    lib.oracle_route_backward.argtypes = [P, P, P, i32, i32, i32, P]
    lib.oracle_backward_mx.restype = i32
    lib.oracle_backward_mx.argtypes = [P, i32, i32, i32, i32, i32, P, P, P, P, P, i32, P, i32, P, i32,
                                       P, P, P, P]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return _load().oracle_num_threads()


def bf16_decode(bits):
    """float32 values of bf16 bit patterns (uint16 array or scalar)."""
    lib = _load()
    b = np.atleast_1d(np.asarray(bits, dtype=np.uint16))
    return np.array([lib.oracle_bf16_decode(int(v)) for v in b.ravel()],
                    dtype=np.float32).reshape(b.shape)


def e4m3_decode(codes):
    lib = _load()
    c = np.atleast_1d(np.asarray(codes, dtype=np.uint8))
    return np.array([lib.oracle_e4m3_decode(int(v)) for v in c.ravel()],
                    dtype=np.float64).reshape(c.shape)


def e4m3_encode(values):
    lib = _load()
    v = np.atleast_1d(np.asarray(values, dtype=np.float32))
    return np.array([lib.oracle_e4m3_encode(float(f)) for f in v.ravel()],
                    dtype=np.uint8).reshape(v.shape)


def quantise_group(values):
    """(codes, scale) of one quantisation group of fp32 values."""
    v = _c(values, np.float32).ravel()
    q = np.empty(v.size, dtype=np.uint8)
    s = _load().oracle_quantise_group(_ptr(v), v.size, _ptr(q))
    return q, np.float32(s)


def router_logits(x_bf16, w_router):
    """fp32 router scores [T, E] = x [T, H] (bf16 bits) times w_router [H, E]
    (fp32), summed in double over ascending h and rounded once."""
    x = _c(x_bf16, np.uint16)
    w = _c(w_router, np.float32)
    T, H = x.shape
    assert w.shape[0] == H
    E = w.shape[1]
    out = np.empty((T, E), np.float32)
    _load().oracle_router_logits(_ptr(x), _ptr(w), T, H, E, _ptr(out))
    return out


def route(logits, k):
    """Top-k routing and its grouped form for fp32 logits [T, E].

    Returns a dict of numpy arrays: topk_ids [T,k] int32, topk_weights [T,k]
    float32, expert_counts [E], expert_offsets [E+1], perm [T*k],
    route_pos [T*k] (all int32)."""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    R = T * k
    out = dict(
        topk_ids=np.empty((T, k), np.int32), topk_weights=np.empty((T, k), np.float32),
        expert_counts=np.empty(E, np.int32), expert_offsets=np.empty(E + 1, np.int32),
        perm=np.empty(R, np.int32), route_pos=np.empty(R, np.int32))
    _load().oracle_route(_ptr(lg), T, E, k, _ptr(out["topk_ids"]), _ptr(out["topk_weights"]),
                         _ptr(out["expert_counts"]), _ptr(out["expert_offsets"]),
                         _ptr(out["perm"]), _ptr(out["route_pos"]))
    return out


def forward(x_bf16, topk_ids, topk_weights, w_gate_up, w_down, quant="bf16",
            s_gate_up=None, s_down=None, tokens=None, expert_begin=0):
    """Layer output (float64 [n_tok, H]) for the listed tokens (all if None).

    x_bf16: uint16 bf16 bits [T,H]; w_gate_up [E,H,2I] and w_down [E,I,H] as
    uint16 bf16 bits (quant "bf16") or uint8 e4m3 codes with fp32 scales:
    per-tensor [E] each, block128 [E,H/128,2I/128] and [E,I/128,H/128].
    Expert-parallel slice: the weights hold experts [expert_begin,
    expert_begin + E) and routes to other experts contribute nothing (the
    per-tensor h scale then covers the local routes only)."""
    q = QUANT[quant]
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    E, H2, I2 = w_gate_up.shape
    assert H2 == H and I2 % 2 == 0
    I = I2 // 2
    k = topk_ids.shape[1]
    wdt = np.uint16 if q == 0 else np.uint8
    wgu = _c(w_gate_up, wdt)
    wd = _c(w_down, wdt)
    assert wd.shape == (E, I, H)
    sdt = np.uint8 if q == 3 else np.float32   # MX: E8M0 scale bytes
    sgu = None if q == 0 else _c(s_gate_up, sdt)
    sd = None if q == 0 else _c(s_down, sdt)
    ids = _c(topk_ids, np.int32)
    tw = _c(topk_weights, np.float32)
    tok = None if tokens is None else _c(tokens, np.int32)
    n_tok = T if tok is None else tok.size
    out = np.zeros((n_tok, H), np.float64)
    rc = _load().oracle_forward_ep(_ptr(x), T, H, I, E, k, _ptr(ids), _ptr(tw), _ptr(wgu), _ptr(wd),
                                   _ptr(sgu), _ptr(sd), q, int(expert_begin), E, _ptr(tok), n_tok,
                                   _ptr(out))
    if rc != 0:
        raise ValueError("oracle_forward rejected the inputs")
    return out


def quantise_activations(x_bf16, quant):
    """(codes uint8 [T,H], scales) of the activation quantisation."""
    q = QUANT[quant]
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    codes = np.empty((T, H), np.uint8)
    if q == 3:
        scales = np.empty(T * (H // 32), np.uint8)
    else:
        scales = np.empty(1 if q == 1 else T * (H // 128), np.float32)
    if _load().oracle_quantise_activations(_ptr(x), T, H, q, _ptr(codes), _ptr(scales)) != 0:
        raise ValueError("unsupported quantisation")
    if q == 3:
        return codes, scales.reshape(T, H // 32)
    return codes, (scales[0] if q == 1 else scales.reshape(T, H // 128))


def gate_up_h(x_bf16, topk_ids, w_gate_up, quant="bf16", s_gate_up=None, routes=None):
    """SwiGLU output h (float64 [n, I]) of the listed route ids r = t*k + j (all
    T*k if None): silu(a W_gate) * (a W_up) with a the token's activation as the
    Gate/Up projection sees it (x quantised for the FP8 formats) -- the tensor
    the Down-input quantisation takes its scales over."""
    q = QUANT[quant]
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    E, H2, I2 = w_gate_up.shape
    assert H2 == H
    I = I2 // 2
    ids = _c(topk_ids, np.int32)
    k = ids.shape[1]
    wgu = _c(w_gate_up, np.uint16 if q == 0 else np.uint8)
    sgu = None if q == 0 else _c(s_gate_up, np.uint8 if q == 3 else np.float32)
    rt = None if routes is None else _c(routes, np.int32)
    n = T * k if rt is None else rt.size
    out = np.zeros((n, I), np.float64)
    if _load().oracle_gate_up_h(_ptr(x), T, H, I, E, k, _ptr(ids), _ptr(wgu), _ptr(sgu), q, _ptr(rt), n,
                                _ptr(out)) != 0:
        raise ValueError("oracle_gate_up_h rejected the inputs")
    return out


def mx_scale_byte(amax):
    """E8M0 byte of an MX group whose largest magnitude is amax (fp32)."""
    return int(_load().oracle_mx_scale_byte(float(np.float32(amax))))


def quantise_group_mx(values):
    """(codes, E8M0 byte) of one MX group of fp32 values."""
    v = _c(values, np.float32).ravel()
    q = np.empty(v.size, dtype=np.uint8)
    b = _load().oracle_quantise_group_mx(_ptr(v), v.size, _ptr(q))
    return q, int(b)


def backward_mx(x_bf16, topk_ids, topk_weights, w_gate_up, w_down, dout_bf16, exact=False,
                tokens=None, experts=None):
    """Gradients of the layer for the upstream gradient dout (bf16 bits [T,H]).

    w_gate_up [E,H,2I] and w_down [E,I,H] are bf16 master weights (uint16
    bits); the MX forward and backward quantise them as each product needs.
    Returns dict(dx [n_tok,H], dgate [n_tok,k], dw_gate_up [n_exp,H,2I],
    dw_down [n_exp,I,H]) in float64 for the listed tokens and experts (all
    when None)."""
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    E, H2, I2 = w_gate_up.shape
    assert H2 == H and I2 % 2 == 0
    I = I2 // 2
    k = topk_ids.shape[1]
    wgu = _c(w_gate_up, np.uint16)
    wd = _c(w_down, np.uint16)
    assert wd.shape == (E, I, H)
    do = _c(dout_bf16, np.uint16)
    assert do.shape == (T, H)
    ids = _c(topk_ids, np.int32)
    tw = _c(topk_weights, np.float32)
    tok = _c(np.arange(T) if tokens is None else tokens, np.int32)
    exps = _c(np.arange(E) if experts is None else experts, np.int32)
    dx = np.zeros((tok.size, H), np.float64)
    dg = np.zeros((tok.size, k), np.float64)
    dwg = np.zeros((exps.size, H, I2), np.float64)
    dwd = np.zeros((exps.size, I, H), np.float64)
    rc = _load().oracle_backward_mx(_ptr(x), T, H, I, E, k, _ptr(ids), _ptr(tw), _ptr(wgu), _ptr(wd),
                                    _ptr(do), int(bool(exact)), _ptr(tok), tok.size, _ptr(exps),
                                    exps.size, _ptr(dx), _ptr(dg), _ptr(dwg), _ptr(dwd))
    if rc != 0:
        raise ValueError("oracle_backward_mx rejected the inputs")
    return {"dx": dx, "dgate": dg, "dw_gate_up": dwg, "dw_down": dwd}


def route_backward(topk_ids, topk_weights, dgate, E):
    """dlogits float64 [T, E] for the gates' upstream gradient dgate [T, k]."""
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    tw = _c(topk_weights, np.float32)
    g = _c(dgate, np.float32)
    out = np.zeros((T, E), np.float64)
    if _load().oracle_route_backward(_ptr(ids), _ptr(tw), _ptr(g), T, E, k, _ptr(out)) != 0:
        raise ValueError("oracle_route_backward rejected the inputs")
    return out
