"""Seeded synthetic inputs for the MoE FFN layer (shared by tests and bench).

This module only draws random inputs and stores them in the formats the layer
consumes; it contains none of the layer's own arithmetic (no routing, no
activation quantisation, no GEMM, no combine).  Both the GPU path and the CPU
oracle receive exactly these arrays.

Recipe (all draws are ``numpy.random.default_rng(seed)`` standard normals):
  * x ~ N(0,1), stored as bf16 (round-to-nearest-even via torch's cast);
  * router logits ~ N(0,1) fp32, or, for the tiny layer, a router weight
    W_r ~ N(0, 0.02) fp32 [H, E] instead (the layer computes its logits x W_r);
  * the prefill-bf16 workload adds a per-expert bias 0.5*ln(1/(e+1)) to its
    logits, giving a Zipf-skewed expert load;
  * expert weights ~ N(0, 0.02), expert e of tensor i drawn from
    default_rng([seed, i, e]) (i = 0 for w_gate_up, 1 for w_down): w_gate_up [E, H, 2I] (gate in columns [0,I),
    up in [I,2I)) and w_down [E, I, H], stored bf16, or quantised offline to
    e4m3 with fp32 scales amax/448 per expert tensor (per-tensor) or per
    128x128 block of the stored [K, N] matrix (block128), or with E8M0
    power-of-two scales per 32 rows of K and output column (MX, fp8_mx32).

Workloads (the shapes of the layers the pages measure):
  tiny_bf16          T=64,   H=256,  I=512, E=16,  k=8  (world-model MoE, E=16 k=8)
  decode_bf16        T=B in 1..4, H=2048, I=768, E=128, k=8 (Qwen3-shaped)
  decode_fp8_tensor  T=B in 1..8, H=4096, I=192, E=192, k=8 (Hunyuan TP8 share)
  prefill_bf16       T=8192, H=2048, I=768, E=128, k=8, Zipf-biased routing
  prefill_fp8_block  T=4096, H=4096, I=512, E=128, k=8, fp8 128x128 blockwise
  prefill_fp8_mx     the same shape, MX fp8 (E8M0 scale per 32 values along K)
  decode_fp8_mx      T=B in 1..8 with prefill_fp8_mx's weights (MX decode)
"""
from __future__ import annotations

import functools
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    quant: str            # "bf16" | "fp8_per_tensor" | "fp8_block128"
    weight_seed: int
    act_seed: int
    logits: str = "normal"  # "normal" | "zipf" | "router"
    batches: tuple = ()


WORKLOADS = {
    "tiny_bf16": Workload("tiny_bf16", 64, 256, 512, 16, 8, "bf16", 1, 1, "router"),
    "decode_bf16": Workload("decode_bf16", 4, 2048, 768, 128, 8, "bf16", 2, 200,
                            batches=(1, 2, 3, 4)),
    "decode_fp8_tensor": Workload("decode_fp8_tensor", 8, 4096, 192, 192, 8, "fp8_per_tensor",
                                  3, 300, batches=(1, 2, 3, 4, 5, 6, 7, 8)),
    # same Qwen3-shaped expert weights as decode_bf16 (one layer, decode and prefill)
    "prefill_bf16": Workload("prefill_bf16", 8192, 2048, 768, 128, 8, "bf16", 2, 4, "zipf"),
    "prefill_fp8_block": Workload("prefill_fp8_block", 4096, 4096, 512, 128, 8, "fp8_block128",
                                  5, 5),
    # the same layer shape with MX FP8 weights (E8M0 scale per 32 values along K)
    "prefill_fp8_mx": Workload("prefill_fp8_mx", 4096, 4096, 512, 128, 8, "fp8_mx32", 7, 5),
    # decode batches over the same MX layer
    "decode_fp8_mx": Workload("decode_fp8_mx", 8, 4096, 512, 128, 8, "fp8_mx32", 7, 700,
                              batches=(1, 2, 3, 4, 5, 6, 7, 8)),
}


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), rounding by torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _e4m3_cast(v: torch.Tensor) -> np.ndarray:
    return torch.clamp(v, -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _scale(amax: torch.Tensor) -> torch.Tensor:
    return torch.where(amax > 0, amax / torch.tensor(448.0, dtype=torch.float32),
                       torch.tensor(1.0, dtype=torch.float32))


def quantise_weight_per_tensor(w: np.ndarray):
    """w [E, K, N] fp32 -> (e4m3 codes, scales [E])."""
    t = torch.from_numpy(w)
    s = _scale(t.abs().amax(dim=(1, 2)))
    return _e4m3_cast(t / s[:, None, None]), s.numpy()


def quantise_weight_block128(w: np.ndarray):
    """w [E, K, N] fp32 -> (e4m3 codes, scales [E, K/128, N/128])."""
    E, K, N = w.shape
    blk = torch.from_numpy(w).view(E, K // 128, 128, N // 128, 128)
    s = _scale(blk.abs().amax(dim=(2, 4)))
    q = _e4m3_cast(blk / s[:, :, None, :, None])
    return q.reshape(E, K, N), s.numpy()


def quantise_weight_mx32(w: np.ndarray):
    """w [E, K, N] fp32 -> (e4m3 codes, E8M0 scale bytes [E, K/32, N]): per 32
    rows of K and output column, scale 2^(floor(log2 amax) - 8) (byte 0 for an
    all-zero group), codes e4m3(w / scale) saturated at 448 (offline weight
    preparation, the MX format's rule)."""
    E, K, N = w.shape
    blk = torch.from_numpy(w).view(E, K // 32, 32, N)
    amax = blk.abs().amax(dim=2)
    _, ex = torch.frexp(amax)
    b = torch.where(amax > 0, (ex - 1 - 8 + 127).clamp(0, 254), torch.zeros_like(ex)).to(torch.int32)
    scale = torch.pow(torch.tensor(2.0, dtype=torch.float64), (b - 127).double()).float()
    q = _e4m3_cast(blk / scale[:, :, None, :])
    return q.reshape(E, K, N), b.to(torch.uint8).numpy()


def _normal_per_expert(shape, seed, tensor_id, std):
    """[E, ...] fp32 draws; expert e uses default_rng([seed, tensor_id, e]) so the
    experts can be drawn on several threads with a fixed result."""
    out = np.empty(shape, np.float32)

    def fill(e):
        rng = np.random.default_rng([seed, tensor_id, e])
        rng.standard_normal(shape[1:], dtype=np.float32, out=out[e])
        out[e] *= np.float32(std)

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, range(shape[0])))
    return out


def random_weights(E, H, I, quant, seed):
    """dict(w_gate_up, w_down, s_gate_up, s_down) for one layer."""
    wgu = _normal_per_expert((E, H, 2 * I), seed, 0, 0.02)
    wd = _normal_per_expert((E, I, H), seed, 1, 0.02)
    if quant == "bf16":
        return dict(w_gate_up=to_bf16_bits(wgu), w_down=to_bf16_bits(wd),
                    s_gate_up=None, s_down=None)
    if quant == "fp8_per_tensor":
        qgu, sgu = quantise_weight_per_tensor(wgu)
        qd, sd = quantise_weight_per_tensor(wd)
    elif quant == "fp8_block128":
        qgu, sgu = quantise_weight_block128(wgu)
        qd, sd = quantise_weight_block128(wd)
    elif quant == "fp8_mx32":
        qgu, sgu = quantise_weight_mx32(wgu)
        qd, sd = quantise_weight_mx32(wd)
    else:
        raise ValueError(quant)
    return dict(w_gate_up=qgu, w_down=qd, s_gate_up=sgu, s_down=sd)


def random_activations(T, H, E, seed, logits="normal"):
    """dict(x bf16 bits [T,H], logits fp32 [T,E]); with logits="router",
    dict(x, w_router fp32 [H,E]) instead."""
    rng = np.random.default_rng(seed)
    x = to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    if logits == "router":
        wr = (rng.standard_normal((H, E)) * 0.02).astype(np.float32)
        return dict(x=x, w_router=wr)
    else:
        lg = rng.standard_normal((T, E), dtype=np.float32)
        if logits == "zipf":
            lg = (lg + (0.5 * np.log(1.0 / np.arange(1, E + 1, dtype=np.float64))
                        ).astype(np.float32)).astype(np.float32)
    return dict(x=x, logits=np.ascontiguousarray(lg, dtype=np.float32))


def random_upstream(T, H, seed):
    """An upstream gradient dout for the layer output: bf16 bits [T, H], unit normal."""
    rng = np.random.default_rng([seed, 7])
    return to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))


@functools.lru_cache(maxsize=2)
def workload_weights(name: str):
    w = WORKLOADS[name]
    return random_weights(w.E, w.H, w.I, w.quant, w.weight_seed)


def workload_inputs(name: str, batch: int | None = None, seed: int | None = None):
    """Activations and logits of a workload; decode workloads take a batch B
    (seed act_seed + B unless given)."""
    w = WORKLOADS[name]
    T = w.T if batch is None else batch
    s = seed if seed is not None else (w.act_seed + (batch or 0) if w.batches else w.act_seed)
    return random_activations(T, w.H, w.E, s, w.logits)


def tie_heavy_logits(T, E, seed):
    """Logits drawn from {-0, +0, 1, 2, 3}: most rows hold exact ties."""
    rng = np.random.default_rng(seed)
    vals = np.array([-0.0, 0.0, 1.0, 2.0, 3.0], dtype=np.float32)
    return vals[rng.integers(0, vals.size, size=(T, E))]
