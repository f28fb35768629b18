"""Pins of the oracle's routing (CPU only).

Top-k is checked against brute force (a full sort of (-logit, id) pairs) and
torch.topk on tie-free rows; gates against torch's float64 softmax; the grouped
form against numpy's stable argsort, its invariants and closed forms.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits_to_f32, random_activations, tie_heavy_logits, to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")


def brute_force_topk(logits, k):
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        # Python float keys: -0.0 == 0.0 compare equal, so ties fall to the id
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))
        ids[t] = order[:k]
    return ids


def check_grouped_form(r, E, k):
    ids = r["topk_ids"].ravel()
    T = r["topk_ids"].shape[0]
    R = T * k
    counts, offs, perm, pos = r["expert_counts"], r["expert_offsets"], r["perm"], r["route_pos"]
    assert counts.sum() == R
    assert offs[0] == 0 and offs[-1] == R
    assert np.array_equal(np.diff(offs), counts)
    assert np.array_equal(np.sort(perm), np.arange(R))
    assert np.array_equal(pos[perm], np.arange(R))
    # expert-major order and stability inside each expert segment
    assert np.all(np.diff(ids[perm]) >= 0)
    for e in range(E):
        seg = perm[offs[e]:offs[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(ids[seg] == e)
    # each token appears exactly k times
    assert np.array_equal(np.bincount(perm // k, minlength=T), np.full(T, k))
    # the library's stable sort gives the same permutation
    assert np.array_equal(perm, np.argsort(ids, kind="stable").astype(np.int32))
    assert np.array_equal(counts, np.bincount(ids, minlength=E))


@pytest.mark.parametrize("T,E,k,seed", [(64, 16, 8, 1), (33, 128, 8, 2), (7, 192, 8, 3),
                                        (100, 5, 1, 4), (50, 64, 64, 5), (3, 512, 20, 6)])
def test_topk_matches_brute_force_and_torch(T, E, k, seed):
    lg = random_activations(T, 8, E, seed)["logits"]
    r = oracle.route(lg, k)
    assert np.array_equal(r["topk_ids"], brute_force_topk(lg, k))
    tv, ti = torch.topk(torch.from_numpy(lg), k, dim=1, sorted=True)
    assert np.array_equal(r["topk_ids"], ti.numpy())   # rows are tie-free (continuous draws)
    check_grouped_form(r, E, k)


@pytest.mark.parametrize("T,E,k,seed", [(200, 16, 8, 10), (64, 128, 8, 11), (40, 7, 7, 12)])
def test_tie_heavy_rows(T, E, k, seed):
    lg = tie_heavy_logits(T, E, seed)
    assert np.any(np.signbit(lg) & (lg == 0))        # the draw holds -0 entries
    r = oracle.route(lg, k)
    assert np.array_equal(r["topk_ids"], brute_force_topk(lg, k))
    check_grouped_form(r, E, k)


def test_negative_zero_ties_with_positive_zero():
    lg = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], np.float32)
    r = oracle.route(lg, 2)
    assert r["topk_ids"].tolist() == [[0, 1], [0, 1]]
    assert np.allclose(r["topk_weights"], 0.5, atol=0)


@pytest.mark.parametrize("T,E,k,seed", [(64, 16, 8, 1), (16, 192, 8, 2), (9, 128, 1, 3)])
def test_gates_match_torch_softmax(T, E, k, seed):
    lg = random_activations(T, 8, E, seed)["logits"]
    r = oracle.route(lg, k)
    p = torch.softmax(torch.from_numpy(lg).double(), dim=1).numpy()
    sel = np.take_along_axis(p, r["topk_ids"].astype(np.int64), axis=1)
    ref = sel / sel.sum(axis=1, keepdims=True)
    assert np.max(np.abs(r["topk_weights"] - ref)) <= 1e-7
    assert np.allclose(r["topk_weights"].sum(axis=1), 1.0, atol=1e-6)
    # slot order is descending logit
    chosen = np.take_along_axis(lg, r["topk_ids"].astype(np.int64), axis=1)
    assert np.all(np.diff(chosen, axis=1) <= 0)


def test_closed_form_single_expert():
    lg = random_activations(37, 8, 1, 5)["logits"]
    r = oracle.route(lg, 1)
    assert np.all(r["topk_ids"] == 0)
    assert np.all(r["topk_weights"] == 1.0)
    assert r["expert_counts"].tolist() == [37]
    assert np.array_equal(r["perm"], np.arange(37))


@pytest.mark.parametrize("T,E", [(5, 16), (3, 64)])
def test_closed_form_all_experts_equal_logits(T, E):
    lg = np.full((T, E), 0.25, np.float32)
    r = oracle.route(lg, E)
    assert np.array_equal(r["topk_ids"], np.tile(np.arange(E, dtype=np.int32), (T, 1)))
    assert np.all(r["topk_weights"] == np.float32(1.0 / E))
    assert np.all(r["expert_counts"] == T)
    assert np.array_equal(r["expert_offsets"], np.arange(E + 1) * T)
    expect = np.array([t * E + e for e in range(E) for t in range(T)], np.int32)
    assert np.array_equal(r["perm"], expect)


def test_empty_batch():
    r = oracle.route(np.zeros((0, 8), np.float32), 2)
    assert r["expert_counts"].tolist() == [0] * 8
    assert r["expert_offsets"].tolist() == [0] * 9
    assert r["perm"].size == 0


def test_golden_hand_example_routing():
    g = json.load(open(GOLDEN))
    r = oracle.route(np.array(g["logits"], np.float32), g["k"])
    ex = g["expected"]
    for key in ("topk_ids", "expert_counts", "expert_offsets", "perm", "route_pos"):
        assert r[key].tolist() == ex[key], key
    assert np.max(np.abs(r["topk_weights"] - np.array(ex["topk_weights"]))) <= ex["tolerance_weights"]


# ------------------------------------------------------------------ router --
def test_router_logits_exact_integer_closed_form():
    """Integer x (exact in bf16) and W_r in multiples of 2^-6: every partial sum is exact in
    double and every score fits fp32's significand, so the scores are the integer matrix product
    (a dropped term, a transposed operand or a wrong index changes them)."""
    rng = np.random.default_rng(40)
    T, H, E = 9, 96, 20
    xi = rng.integers(-16, 17, size=(T, H))
    wi = rng.integers(-128, 129, size=(H, E))
    x_bits = to_bf16_bits(xi.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f32(x_bits), xi.astype(np.float32))
    got = oracle.router_logits(x_bits, (wi / 64.0).astype(np.float32))
    assert np.array_equal(got.astype(np.float64) * 64.0, (xi @ wi).astype(np.float64))


def test_router_logits_one_hot_columns_select_activations():
    T, H, E = 5, 64, 24
    x_bits = random_activations(T, H, E, 41)["x"]
    cols = np.random.default_rng(42).choice(H, E, replace=False)
    w = np.zeros((H, E), np.float32)
    w[cols, np.arange(E)] = 1.0
    assert np.array_equal(oracle.router_logits(x_bits, w), bf16_bits_to_f32(x_bits)[:, cols])


def test_router_logits_match_float64_product():
    """numpy's float64 product (another summation order) rounded to fp32: at most one fp32 ulp
    apart, and almost always identical."""
    a = random_activations(64, 256, 16, 1, logits="router")
    got = oracle.router_logits(a["x"], a["w_router"])
    ref = (bf16_bits_to_f32(a["x"]).astype(np.float64) @ a["w_router"].astype(np.float64)).astype(np.float32)
    ulps = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1 and np.mean(ulps == 0) >= 0.99
