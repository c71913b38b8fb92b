"""Pins for the oracle's gate: logits, top-k selection and routing weights.

The oracle is checked here against things other than itself: float64 dot
products with the float32 summation error bound, a constructed case whose
float32 result depends on the summation order, brute force over every k-subset
with the exact ranking predicate, numpy's stable argsort, torch's softmax, and
a tiny routing example worked by hand (tests/golden/routing_tiny.json).
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from moe_workloads import bf16_bits_to_f32, to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(a):
    return a.astype(np.float64) if a.dtype == np.float32 else bf16_bits_to_f32(a).astype(np.float64)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_logits_within_float32_error_bound(act):
    rng = np.random.default_rng(11)
    T, d, E = 48, 333, 12
    x = rng.standard_normal((T, d), dtype=np.float32)
    wg = (rng.standard_normal((E, d), dtype=np.float32) * 0.02).astype(np.float32)
    bias = rng.standard_normal(E).astype(np.float32)
    if act == "bf16":
        x, wg = to_bf16_bits(x), to_bf16_bits(wg)
    z = oracle.gate_logits(x, wg, bias).astype(np.float64)
    X, W = _f64(x), _f64(wg)
    exact = X @ W.T
    mag = np.abs(X) @ np.abs(W).T
    u = 2.0 ** -24
    gamma = (d + 1) * u / (1 - (d + 1) * u)
    bound = gamma * (mag + np.abs(bias)[None, :]) + 2 * u * np.abs(exact + bias[None, :])
    err = np.abs(z - (exact + bias[None, :]))
    assert np.all(err <= bound), float((err / np.maximum(bound, 1e-300)).max())
    # a dropped bias or a transposed operand is far outside the bound
    assert np.abs(exact).max() > 10 * bound.max()


def test_logits_sum_order_is_one_ascending_chain():
    # 1 + 2^26 rounds back to 2^26 in float32, so the ascending chain gives 0
    # while the exact sum is 1; with the large terms first the chain gives 1.
    wg = np.ones((1, 3), dtype=np.float32)
    small_first = np.array([[1.0, 2.0 ** 26, -(2.0 ** 26)]], dtype=np.float32)
    large_first = np.array([[2.0 ** 26, -(2.0 ** 26), 1.0]], dtype=np.float32)
    assert oracle.gate_logits(small_first, wg)[0, 0] == 0.0
    assert oracle.gate_logits(large_first, wg)[0, 0] == 1.0
    # the same holds in bf16 storage (all three values are exact in bf16)
    assert oracle.gate_logits(to_bf16_bits(small_first), to_bf16_bits(wg))[0, 0] == 0.0


def test_logits_exact_on_small_integers():
    rng = np.random.default_rng(5)
    x = rng.integers(-8, 9, size=(20, 64)).astype(np.float32)
    wg = rng.integers(-8, 9, size=(7, 64)).astype(np.float32)
    z = oracle.gate_logits(x, wg)
    assert np.array_equal(z.astype(np.int64), x.astype(np.int64) @ wg.astype(np.int64).T)


def _brute_force_topk(z, k):
    E = len(z)
    winners = []
    for sub in itertools.combinations(range(E), k):
        s = set(sub)
        ok = all(z[i] > z[j] or (z[i] == z[j] and i < j)
                 for i in s for j in range(E) if j not in s)
        if ok:
            winners.append(s)
    assert len(winners) == 1
    return winners[0]


@pytest.mark.parametrize("seed", range(6))
def test_selection_brute_force_with_ties(seed):
    rng = np.random.default_rng(100 + seed)
    for _ in range(40):
        E = int(rng.integers(1, 11))
        k = int(rng.integers(1, E + 1))
        # a coarse grid makes ties frequent
        z = (np.round(rng.standard_normal(E) * 2) / 2).astype(np.float32)
        idx, w = oracle.select_topk(z[None, :], k)
        assert set(idx[0].tolist()) == _brute_force_topk(z, k)
        # descending key order, ties to lower id == numpy's stable argsort of -z
        assert idx[0].tolist() == np.argsort(-z, kind="stable")[:k].tolist()


@pytest.mark.parametrize("E,k", [(6, 2), (16, 4), (200, 8)])
def test_nan_logits_rank_after_every_number(E, k):
    # numpy's stable sort puts NaN after every number and keeps equal keys
    # (NaNs included) in index order: the ranking the selection must follow
    rng = np.random.default_rng(E)
    z = (np.round(rng.standard_normal((300, E)) * 2) / 2).astype(np.float32)
    z[rng.random((300, E)) < 0.2] = np.nan
    z[5, :] = np.nan                 # every logit NaN
    z[6, : E - k + 1] = np.nan       # fewer than k numbers
    z[7, 1] = np.inf
    z[8, :] = -np.inf
    z[8, 3] = np.nan
    idx, w = oracle.select_topk(z, k)
    for t in range(len(z)):
        assert idx[t].tolist() == np.argsort(-z[t], kind="stable")[:k].tolist(), t
    # a NaN logit has probability 0; the numbers share the weight
    sel = np.take_along_axis(z, idx, axis=1)
    nan_sel = np.isnan(sel)
    ok = ~np.all(nan_sel | (sel == -np.inf), axis=1) & ~np.any(sel == np.inf, axis=1)
    assert np.all(w[ok][nan_sel[ok]] == 0.0)
    ref = torch.softmax(torch.from_numpy(np.where(nan_sel, -np.inf, sel).astype(np.float64)), -1)
    np.testing.assert_allclose(w[ok], ref.numpy()[ok], rtol=1e-12, atol=1e-300)
    # no number to give the weight to: NaN weights
    assert np.all(np.isnan(w[5])) and np.all(np.isnan(w[8]))


def test_ties_go_to_lower_expert_id():
    rng = np.random.default_rng(3)
    d = 32
    base = rng.standard_normal((4, d), dtype=np.float32)
    wg = np.stack([base[0], base[1], base[0], base[1], base[2], base[0]])  # duplicated rows
    x = rng.standard_normal((64, d), dtype=np.float32)
    idx, _, z = oracle.gate_topk(x, wg, k=3)
    for t in range(64):
        assert z[t, 0] == z[t, 2] == z[t, 5] and z[t, 1] == z[t, 3]
        chosen = idx[t].tolist()
        # among equal logits the lower id is always taken first
        for a, b in ((0, 2), (2, 5), (1, 3)):
            if b in chosen:
                assert a in chosen and chosen.index(a) < chosen.index(b)


def test_weights_match_topk_then_softmax_form():
    # renormalised full softmax (wmrh.cn 4.1) == softmax of the k selected
    # logits (lpnh.cn chapter 1, top2_gating)
    rng = np.random.default_rng(8)
    z = rng.standard_normal((200, 16)).astype(np.float32) * 3
    for k in (1, 2, 4, 7):
        idx, w = oracle.select_topk(z, k)
        sel = torch.from_numpy(np.take_along_axis(z, idx, axis=1).astype(np.float64))
        ref = torch.softmax(sel, dim=-1).numpy()
        np.testing.assert_allclose(w, ref, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=8 * k * 2.0 ** -52)
        assert np.all(np.diff(w, axis=1) <= 0)  # rank order
        if k == 1:
            assert np.all(w == 1.0)


def test_k_equals_E_is_the_full_softmax():
    rng = np.random.default_rng(9)
    z = rng.standard_normal((50, 9)).astype(np.float32)
    idx, w = oracle.select_topk(z, 9)
    full = torch.softmax(torch.from_numpy(z.astype(np.float64)), dim=-1).numpy()
    np.testing.assert_allclose(w, np.take_along_axis(full, idx, axis=1), rtol=1e-12, atol=0)


def test_golden_tiny_routing():
    g = json.load(open(os.path.join(GOLDEN, "routing_tiny.json")))
    x = np.array(g["x"], dtype=np.float32)
    wg = np.array(g["w_gate"], dtype=np.float32)
    idx, w, z = oracle.gate_topk(x, wg, g["k"])
    assert np.array_equal(z, np.array(g["logits"], dtype=np.float32))
    assert idx.tolist() == g["topk_idx"]
    closed = [[0.5, 0.5], [1 / (1 + math.exp(-0.5)), 1 - 1 / (1 + math.exp(-0.5))],
              [0.5, 0.5], [1 / (1 + math.exp(-1)), 1 - 1 / (1 + math.exp(-1))]]
    np.testing.assert_allclose(w, closed, rtol=1e-14)
    np.testing.assert_allclose(w, g["topk_w"], rtol=1e-14)
    counts, offsets, dest, src = oracle.dispatch(idx, wg.shape[0])
    assert counts.tolist() == g["counts"] and offsets.tolist() == g["offsets"]
    assert dest.tolist() == g["dest_row"] and src.tolist() == g["src_token"]
