"""Pins for the oracle's expert FFN, layer composition and combine.

SwiGLU here is W2 (silu(W1 v) * (W3 v)). The layer is pinned by reductions
to a dense FFN computed with float64 numpy matmuls: one expert with k=1;
identical experts (the gate weights sum to one, so routing must not matter);
routed experts zeroed (only the shared experts remain); and the fp8 path,
where only the routed experts see the dequantised row. Combine is pinned by a
payload whose every row carries its source token id.
"""

import numpy as np
import pytest

import oracle
from moe_workloads import CONFIGS, MoEInputs, bf16_bits_to_f32, make_inputs, make_weights


def _w64(a):
    return a.astype(np.float64) if a.dtype == np.float32 else bf16_bits_to_f32(a).astype(np.float64)


def dense_swiglu(v, w1, w3, w2):
    a = v @ _w64(w1).T
    b = v @ _w64(w3).T
    return (a / (1.0 + np.exp(-a)) * b) @ _w64(w2).T


def _small(act="f32", T=40, d=32, E=4, k=2, S=0, h=24, fp8=False, seed=0):
    base = CONFIGS["tiny_fp32" if act == "f32" else "deepseekmoe_bf16"]
    import dataclasses
    cfg = dataclasses.replace(base, T=T, d=d, E=E, k=k, S=S, h=h, sigma_w=0.2,
                              dispatch="fp8" if fp8 else "act")
    return make_inputs(cfg, seed=seed)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_single_expert_is_a_dense_swiglu(act):
    inp = _small(act, E=1, k=1)
    idx, w, y = oracle.layer_tokens(inp, np.arange(inp.cfg.T))
    assert np.all(idx == 0) and np.all(w == 1.0)
    ref = dense_swiglu(_w64(inp.x), inp.w1[0], inp.w3[0], inp.w2[0])
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_identical_experts_make_routing_irrelevant(act):
    inp = _small(act, E=6, k=3, S=0)
    for g in range(1, 6):
        inp.w1[g], inp.w3[g], inp.w2[g] = inp.w1[0], inp.w3[0], inp.w2[0]
    _, _, y = oracle.layer_tokens(inp, np.arange(inp.cfg.T))
    ref = dense_swiglu(_w64(inp.x), inp.w1[0], inp.w3[0], inp.w2[0])
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)


def test_shared_experts_only_when_routed_outputs_are_zero():
    inp = _small("bf16", E=5, k=2, S=2)
    inp.w2[:5] = 0
    _, _, y = oracle.layer_tokens(inp, np.arange(inp.cfg.T))
    v = _w64(inp.x)
    ref = dense_swiglu(v, inp.w1[5], inp.w3[5], inp.w2[5]) + dense_swiglu(v, inp.w1[6], inp.w3[6], inp.w2[6])
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)


def test_fp8_applies_to_routed_experts_only():
    inp = _small("bf16", E=3, k=2, S=1, fp8=True, d=64)
    for g in range(1, 4):
        inp.w1[g], inp.w3[g], inp.w2[g] = inp.w1[0], inp.w3[0], inp.w2[0]
    _, _, y = oracle.layer_tokens(inp, np.arange(inp.cfg.T))
    q, qp = oracle.fp8_quantize(inp.x)
    dq = oracle.fp8_dequantize(q, qp)
    ref = dense_swiglu(_w64(inp.x), inp.w1[0], inp.w3[0], inp.w2[0]) + \
        dense_swiglu(dq, inp.w1[0], inp.w3[0], inp.w2[0])
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)
    # and it does differ from the unquantised layer
    assert np.abs(dq - _w64(inp.x)).max() > 0


def test_expert_rows_match_numpy():
    inp = _small("bf16", E=4, k=2, S=1)
    rng = np.random.default_rng(2)
    rows = rng.standard_normal((10, inp.cfg.d))
    group = rng.integers(0, 5, 10).astype(np.int32)
    out = oracle.expert_rows(rows, group, inp.w1, inp.w3, inp.w2)
    for r in range(10):
        g = group[r]
        np.testing.assert_allclose(out[r], dense_swiglu(rows[r:r + 1], inp.w1[g], inp.w3[g], inp.w2[g])[0],
                                   rtol=1e-11, atol=1e-13)


def test_layer_selection_matches_gate():
    inp = _small("bf16", T=64, E=8, k=3, S=1)
    idx, w, _ = oracle.layer_tokens(inp, np.arange(64))
    idx2, w2, _ = oracle.gate_topk(inp.x, inp.wg, 3)
    assert np.array_equal(idx, idx2) and np.array_equal(w, w2)


@pytest.mark.parametrize("with_shared", [False, True])
def test_combine_source_token_payload(with_shared):
    T, E, k, d = 200, 16, 4, 8
    from moe_workloads import make_routing
    idx = make_routing(T, E, k, seed=7)
    _, _, dest, src = oracle.dispatch(idx, E)
    y_perm = np.repeat(src.astype(np.float32)[:, None], d, axis=1)
    w = make_weights(T, k)
    ys = np.full((T, d), 0.5, dtype=np.float32) if with_shared else None
    y = oracle.combine(y_perm, ys, dest, w)
    expect = np.arange(T, dtype=np.float64)[:, None] * w.astype(np.float64).sum(axis=1, keepdims=True)
    expect = np.repeat(expect, d, axis=1) + (0.5 if with_shared else 0.0)
    np.testing.assert_allclose(y, expect, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y - (0.5 if with_shared else 0.0),
                               np.repeat(np.arange(T)[:, None], d, axis=1), rtol=2e-6, atol=1e-4)


def test_combine_k1_is_a_pure_unpermute():
    T, E, d = 64, 8, 4
    from moe_workloads import make_routing
    idx = make_routing(T, E, 1, seed=9)
    _, _, dest, src = oracle.dispatch(idx, E)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((T, d)).astype(np.float32)
    y = oracle.combine(x[src], None, dest, np.ones((T, 1), dtype=np.float32))
    assert np.array_equal(y, x.astype(np.float64))


def test_layer_route():
    # the top-k as route: the plain layer; every slot dropped and no shared
    # experts: zero; with identical experts, dropping one slot of every
    # token leaves (1 - w_dropped) of the dense FFN, and moving a slot to
    # another (identical) expert changes nothing
    inp = _small("f32", E=6, k=3, S=0)
    toks = np.arange(inp.cfg.T)
    idx, w, y = oracle.layer_tokens(inp, toks)
    _, _, y_same = oracle.layer_tokens(inp, toks, route=idx)
    assert np.array_equal(y_same, y)
    _, _, y_none = oracle.layer_tokens(inp, toks, route=np.full_like(idx, -1))
    assert np.all(y_none == 0)
    # a route to a different expert computes that expert's FFN
    moved = idx.copy()
    moved[:, 0] = (idx[:, 0] + 1) % 6
    _, _, y_moved = oracle.layer_tokens(inp, toks, route=moved)
    v = _w64(inp.x)
    ref = sum(w[:, j:j + 1] * np.stack([dense_swiglu(v[t:t + 1], inp.w1[g], inp.w3[g], inp.w2[g])[0]
                                         for t, g in enumerate(moved[:, j])])
              for j in range(3))
    np.testing.assert_allclose(y_moved, ref, rtol=1e-10, atol=1e-12)
    for g in range(1, 6):
        inp.w1[g], inp.w3[g], inp.w2[g] = inp.w1[0], inp.w3[0], inp.w2[0]
    drop = idx.copy()
    drop[:, 1] = -1
    _, w, y_drop = oracle.layer_tokens(inp, toks, route=drop)
    ref = dense_swiglu(v, inp.w1[0], inp.w3[0], inp.w2[0]) * (1.0 - w[:, 1:2])
    np.testing.assert_allclose(y_drop, ref, rtol=1e-10, atol=1e-12)


def test_layer_qrange_own_range_is_the_default():
    inp = _small("bf16", E=6, k=2, S=1, fp8=True)
    toks = np.arange(inp.cfg.T)
    _, _, y = oracle.layer_tokens(inp, toks)
    xf = bf16_bits_to_f32(inp.x)
    own = np.stack([xf.min(1), xf.max(1)], 1).astype(np.float32)
    qr = np.repeat(own[:, None, :], 2, axis=1)
    _, _, y2 = oracle.layer_tokens(inp, toks, qrange=qr)
    assert np.array_equal(y, y2)
    # a wider range changes the routed experts' input only
    wide = qr.copy()
    wide[..., 0] -= 4.0
    _, _, y3 = oracle.layer_tokens(inp, toks, qrange=wide)
    assert not np.array_equal(y, y3)
