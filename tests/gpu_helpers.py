"""Shared helpers of the GPU parity tests: move seeded host inputs to the GPU,
run the layer through the C ABI, and compare with the CPU oracle."""
import functools

import numpy as np
import torch

import oracle
import routing_grouped_expert_index_amd as moe
from workloads import WORKLOADS, random_activations, random_weights, workload_inputs, workload_weights

DEV = torch.device("cuda:0")

TOL = {"bf16": dict(max_abs=2e-2, rel_l2=1e-2), "fp8": dict(rel_l2=2e-2, cos=0.999)}


def say(msg):
    print(msg, flush=True)


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def weights_dev(w: dict, quant: str):
    """Packed device weights and scales from host weights."""
    if quant == "bf16":
        gu = torch.from_numpy(w["w_gate_up"].view(np.int16)).to(DEV)
        dn = torch.from_numpy(w["w_down"].view(np.int16)).to(DEV)
        scales = None
    else:
        gu = torch.from_numpy(w["w_gate_up"]).to(DEV)
        dn = torch.from_numpy(w["w_down"]).to(DEV)
        scales = (torch.from_numpy(w["s_gate_up"]).to(DEV), torch.from_numpy(w["s_down"]).to(DEV))
        if quant == "fp8_mx32":
            scales = moe.pack_mx_scales(*scales)
    pw = moe.pack_weights(gu, dn, quant)
    torch.cuda.synchronize()
    del gu, dn
    return pw, scales


@functools.lru_cache(maxsize=1)
def workload_dev(name: str):
    w = workload_weights(name)
    return weights_dev(w, WORKLOADS[name].quant)


def run(x_bits, logits, k, dev_w, quant, path="auto"):
    pw, scales = dev_w
    r = moe.route(torch.from_numpy(np.ascontiguousarray(logits)).to(DEV), k)
    out = moe.forward(bf16_dev(x_bits), r, pw, quant=quant, scales=scales, path=path)
    torch.cuda.synchronize()
    return r, out


def routes_np(r):
    return dict(topk_ids=r.topk_ids.cpu().numpy(), topk_weights=r.topk_weights.cpu().numpy(),
                expert_counts=r.expert_counts.cpu().numpy(), expert_offsets=r.expert_offsets.cpu().numpy(),
                perm=r.perm.cpu().numpy(), route_pos=r.route_pos.cpu().numpy())


def check_routing(got: dict, ref: dict):
    for key in ("topk_ids", "expert_counts", "expert_offsets", "perm", "route_pos"):
        assert np.array_equal(got[key].reshape(ref[key].shape), ref[key]), f"routing {key} differs"
    if ref["topk_weights"].size:
        d = np.max(np.abs(got["topk_weights"] - ref["topk_weights"]))
        assert d <= 1e-6, f"gates differ by {d}"


def metrics(got: np.ndarray, ref: np.ndarray):
    got = got.astype(np.float64)
    diff = got - ref
    nref = np.linalg.norm(ref)
    return dict(max_abs=float(np.max(np.abs(diff))) if diff.size else 0.0,
                rel_l2=float(np.linalg.norm(diff) / nref) if nref > 0 else float(np.linalg.norm(diff)),
                cos=float(np.dot(got.ravel(), ref.ravel()) / (np.linalg.norm(got) * nref))
                if nref > 0 and np.linalg.norm(got) > 0 else 1.0)


def check_out(got: np.ndarray, ref: np.ndarray, quant: str, what=""):
    m = metrics(got, ref)
    say(f"  {what}: max-abs {m['max_abs']:.3e} rel-L2 {m['rel_l2']:.3e} cos {m['cos']:.6f}")
    if quant == "bf16":
        assert m["max_abs"] <= TOL["bf16"]["max_abs"] and m["rel_l2"] <= TOL["bf16"]["rel_l2"], (what, m)
    else:
        assert m["rel_l2"] <= TOL["fp8"]["rel_l2"] and m["cos"] >= TOL["fp8"]["cos"], (what, m)
    return m


def oracle_out(x_bits, ref_routes, w, quant, tokens=None):
    return oracle.forward(x_bits, ref_routes["topk_ids"], ref_routes["topk_weights"], w["w_gate_up"],
                          w["w_down"], quant=quant, s_gate_up=w["s_gate_up"], s_down=w["s_down"],
                          tokens=tokens)


__all__ = ["DEV", "say", "bf16_dev", "weights_dev", "workload_dev", "run", "routes_np", "check_routing",
           "check_out", "oracle_out", "metrics", "random_activations", "random_weights", "workload_inputs",
           "workload_weights", "WORKLOADS", "oracle", "moe"]


