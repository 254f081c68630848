"""Pins of the oracle's fp32 programs and routing (CPU only).

The fp32 programs (tree_sum, the router chain, exp_p) are fixed by hand-worked
fixtures that separate them from nearby alternatives (another summation order,
a non-fused product), and bounded against binary64 / libm.  Top-k and the
permutation are checked against numpy's stable sorts.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from conftest import read_golden, ulp_diff_f32

U = 2.0 ** -24   # unit roundoff of fp32


def _f(vals):
    return np.array([float(v) for v in vals], dtype=np.float32)


# ---------------------------------------------------------------- summation
def test_tree_sum_golden():
    g = read_golden("summation_order.txt")
    assert oracle.tree_sum(_f(g["tree_in"])) == np.float32(g["tree_out"][0])
    assert oracle.tree_sum(_f(g["tree3_in"])) == np.float32(g["tree3_out"][0])


def test_tree_sum_exact_and_bounded():
    rng = np.random.default_rng(0)
    for n in [1, 2, 3, 5, 31, 64, 100]:
        ints = rng.integers(-1000, 1000, n).astype(np.float32)   # exact sums
        assert oracle.tree_sum(ints) == np.float32(ints.astype(np.int64).sum())
        v = rng.standard_normal(n).astype(np.float32)
        err = abs(float(oracle.tree_sum(v)) - float(np.sum(v.astype(np.float64))))
        assert err <= math.ceil(math.log2(max(n, 2))) * U * np.abs(v).astype(np.float64).sum() * 1.01


def test_router_chain_golden():
    g = read_golden("summation_order.txt")
    # one chunk, sequential fused chain
    x = np.zeros((1, 32), np.float32)
    W = np.zeros((32, 1), np.float32)
    x[0, :4], W[:4, 0] = _f(g["chain_x"]), _f(g["chain_w"])
    assert oracle.router_logits(x, W)[0, 0] == np.float32(g["chain_out"][0])
    # fused multiply-add keeps the exact product
    x = np.zeros((1, 32), np.float32)
    W = np.zeros((32, 1), np.float32)
    x[0, :2], W[:2, 0] = _f(g["fma_x"]), _f(g["fma_w"])
    assert oracle.router_logits(x, W)[0, 0] == np.float32(float(g["fma_out"][0]))
    # chunk partials summed by the tree, bias added afterwards
    x = np.zeros((1, 128), np.float32)
    W = np.zeros((128, 1), np.float32)
    x[0, ::32] = _f(g["chunks_partials"])
    W[::32, 0] = 1.0
    assert oracle.router_logits(x, W)[0, 0] == np.float32(g["chunks_out"][0])
    b = _f(g["chunks_bias"])
    assert oracle.router_logits(x, W, b)[0, 0] == np.float32(g["chunks_out_bias"][0])


@pytest.mark.parametrize("T,H,E", [(5, 256, 8), (3, 2048, 128), (2, 96, 3)])
def test_router_vs_binary64(T, H, E):
    rng = np.random.default_rng(T * H + E)
    x = rng.standard_normal((T, H)).astype(np.float32)
    W = (rng.standard_normal((H, E)) * 0.02).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    got = oracle.router_logits(x, W, b).astype(np.float64)
    ref = x.astype(np.float64) @ W.astype(np.float64) + b
    mag = np.abs(x.astype(np.float64)) @ np.abs(W.astype(np.float64)) + np.abs(b)
    depth = 32 + math.ceil(math.log2(max(H // 32, 2))) + 1
    assert np.all(np.abs(got - ref) <= depth * U * mag * 1.01)


# ---------------------------------------------------------------- exp_p, silu
def test_exp_p_accuracy():
    xs = np.concatenate([
        np.linspace(-103.9, 88.7, 400_001, dtype=np.float32),
        np.linspace(-1, 1, 100_001, dtype=np.float32),
        np.array([0.0, -0.0, 1e-30, -1e-30, 88.72, -87.33, -88.0], np.float32)])
    got = oracle.exp_p(xs)
    ref = np.exp(xs.astype(np.float64))
    normal = ref >= 2.0 ** -126
    ref32 = ref.astype(np.float32)
    fin = normal & np.isfinite(ref32)
    # within 2 ulp of the correctly rounded value wherever the result is normal
    assert ulp_diff_f32(got[fin], ref32[fin]).max() <= 2
    # subnormal results: within 2 units of 2^-149
    sub = ~normal
    assert np.all(np.abs(got[sub].astype(np.float64) - ref[sub]) <= 2 * 2.0 ** -149)


def test_exp_p_special_values():
    v = oracle.exp_p([0.0, 89.0, 200.0, -104.0, -1000.0, 1.0])
    assert v[0] == 1.0 and np.isinf(v[1]) and np.isinf(v[2])
    assert v[3] == 0.0 and v[4] == 0.0
    assert abs(float(v[5]) - math.e) <= 2 * U * math.e


def test_silu_p_accuracy():
    g = np.linspace(-30, 30, 120_001, dtype=np.float32)
    got = oracle.silu_p(g).astype(np.float64)
    gd = g.astype(np.float64)
    ref = gd / (1.0 + np.exp(-gd))
    assert np.all(np.abs(got - ref) <= 6 * U * np.abs(ref) + 1e-45)


# ---------------------------------------------------------------- top-k
def _brute_topk(logits, k):
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))
        ids[t] = order[:k]
    return ids


@pytest.mark.parametrize("E,k", [(8, 2), (128, 8), (256, 8), (5, 5), (3, 1)])
def test_topk_vs_sort(E, k):
    rng = np.random.default_rng(E * 31 + k)
    logits = rng.standard_normal((200, E)).astype(np.float32)
    logits[:20] = np.round(logits[:20] * 2) / 2          # many exact ties
    logits[20] = 0.0                                     # all tied
    ids, w32, w64 = oracle.topk(logits, k)
    assert np.array_equal(ids, _brute_topk(logits, k))
    assert list(ids[20]) == list(range(k))
    sel = np.take_along_axis(logits, ids, axis=1).astype(np.float64)
    assert np.allclose(w64, softmax(sel, axis=1), rtol=1e-14, atol=0)
    assert np.all(np.abs(w32.astype(np.float64) - w64) <= 8 * U * w64 + 1e-45)
    assert np.all(np.abs(w32.astype(np.float64).sum(1) - 1.0) <= 2 * k * U)


def test_topk_single_expert_weight_is_one():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((50, 16)).astype(np.float32)
    _, w32, w64 = oracle.topk(logits, 1)
    assert np.all(w32 == 1.0) and np.all(w64 == 1.0)


def test_topk_negative_zero_ties_lower_index():
    logits = np.array([[-0.0, 0.0, -1.0, 0.0]], np.float32)
    ids, _, _ = oracle.topk(logits, 3)
    assert list(ids[0]) == [0, 1, 3]


def test_router_duplicate_columns_tie():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    W = (rng.standard_normal((256, 8)) * 0.02).astype(np.float32)
    W[:, 5] = W[:, 2]                                    # experts 2 and 5 tie exactly
    logits = oracle.router_logits(x, W)
    assert np.array_equal(logits[:, 2].view(np.uint32), logits[:, 5].view(np.uint32))
    ids, _, _ = oracle.topk(logits, 8)
    pos = {e: np.argmax(ids == e, axis=1) for e in (2, 5)}
    assert np.all(pos[2] + 1 == pos[5])                  # lower index first, adjacent


# ---------------------------------------------------------------- permutation
@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (513, 128, 8), (40, 256, 8), (7, 1, 1)])
def test_permutation_vs_stable_argsort(T, E, k):
    rng = np.random.default_rng(T + E)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, inv = oracle.route_permutation(ids, E)
    assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(perm, np.argsort(ids.ravel(), kind="stable"))
    assert np.array_equal(inv[perm], np.arange(T * k))
    for e in range(E):                                   # ascending token per segment
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(ids.ravel()[seg] == e)
        assert np.all(np.diff(seg // k) > 0)


def test_permutation_empty():
    ids = np.zeros((0, 2), np.int32)
    counts, offsets, perm, inv = oracle.route_permutation(ids, 4)
    assert counts.sum() == 0 and np.all(offsets == 0) and perm.size == 0
