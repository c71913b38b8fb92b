"""Pins for the oracle's whole-batch expert stage (oracle/dense.py).

The whole-batch form applies each expert to all of its rows with one
float64 matrix product; the per-token C oracle (layer_tokens, expert_rows)
applies it to one row at a time with scalar loops. The two share no
arithmetic code, so agreement to float64 rounding on small cases of every
workload kind -- float32 and bf16 activations, shared experts, the Zipf gate
offset, fp8 rows, a capacity limit with dropped and reassigned slots, and
the per-expert fp8 ranges -- pins the whole-batch form to the per-token one,
which is itself pinned to dense SwiGLU reductions and closed forms
(test_oracle_ffn.py).
"""

import dataclasses

import numpy as np
import pytest

import oracle
from moe_workloads import CONFIGS, make_inputs

# float64 sums in a different order: a few ulps of the result's scale
REL = 1e-12


def _cfg(name, **kw):
    base = dict(T=300, d=256, h=96)
    base.update(kw)
    return dataclasses.replace(CONFIGS[name], **base)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("name,kw", [
    ("tiny_fp32", dict(T=256, d=64, h=128)),
    ("deepseekmoe_bf16", {}),
    ("coarse_top2_bf16", {}),
    ("zipf_stress_bf16", {}),
    ("fp8_dispatch", {}),
    ("fp8_dispatch", dict(T=77, d=48, h=40, E=5, k=5, S=1)),
])
def test_layer_matches_per_token_oracle(name, kw):
    cfg = _cfg(name, **kw)
    inp = make_inputs(cfg, seed=4)
    idx, w, y = oracle.layer_tokens(inp, np.arange(cfg.T), nthreads=4)
    i2, w2, y2 = oracle.layer_dense(inp, nthreads=4, chunk=64)
    assert np.array_equal(idx, i2)
    assert np.array_equal(w, w2)
    assert _rel(y2, y) <= REL
    # per token too
    for t in range(0, cfg.T, 37):
        assert _rel(y2[t], y[t]) <= 1e-11


@pytest.mark.parametrize("reassign", [False, True])
def test_layer_with_capacity_route(reassign):
    cfg = _cfg("zipf_stress_bf16", T=256, d=128, h=64, E=16, k=4)
    inp = make_inputs(cfg, seed=5)
    z = oracle.gate_logits(inp.x, inp.wg, inp.bias)
    idx, w = oracle.select_topk(z, cfg.k)
    cap = cfg.T * cfg.k // cfg.E
    *_, route = oracle.dispatch(idx, cfg.E, capacity=cap, reassign=reassign, return_route=True)
    assert np.any(route != idx)
    if reassign:
        # a reassigned slot can land on an expert its token already has
        dup = any(len(set(r[r >= 0].tolist())) < int((r >= 0).sum()) for r in route)
        assert dup, "this case should exercise a token holding one expert twice"
    else:
        assert np.any(route < 0)
    _, _, y = oracle.layer_tokens(inp, np.arange(cfg.T), route=route)
    _, _, y2 = oracle.layer_dense(inp, route=route, chunk=40)
    assert _rel(y2, y) <= REL


def test_layer_with_fp8_expert_ranges():
    cfg = _cfg("fp8_dispatch", T=120, d=64, h=32, E=6, k=2, S=1)
    inp = make_inputs(cfg, seed=6)
    z = oracle.gate_logits(inp.x, inp.wg)
    idx, _ = oracle.select_topk(z, cfg.k)
    xf = (inp.x.astype(np.uint32) << 16).view(np.float32)
    lo = np.array([xf[np.any(idx == e, axis=1)].min() if np.any(idx == e) else 0 for e in range(cfg.E)])
    hi = np.array([xf[np.any(idx == e, axis=1)].max() if np.any(idx == e) else 0 for e in range(cfg.E)])
    qrange = np.stack([lo[idx], hi[idx]], axis=-1).astype(np.float32)
    _, _, y = oracle.layer_tokens(inp, np.arange(cfg.T), qrange=qrange)
    _, _, y2 = oracle.layer_dense(inp, qrange=qrange, chunk=30)
    assert _rel(y2, y) <= REL


@pytest.mark.parametrize("name", ["deepseekmoe_bf16", "fp8_dispatch"])
def test_routed_and_shared_rows_match_expert_rows(name):
    cfg = _cfg(name, T=150, d=128, h=64, E=8, k=3)
    inp = make_inputs(cfg, seed=7)
    z = oracle.gate_logits(inp.x, inp.wg, inp.bias)
    idx, _ = oracle.select_topk(z, cfg.k)
    counts, offsets, dest, src = oracle.dispatch(idx, cfg.E)
    R = int(offsets[-1])
    got = np.zeros((R, cfg.d))
    seen = np.zeros(R, dtype=bool)
    for r0, r1, out in oracle.routed_rows(inp, offsets, src, chunk=17,
                                          xq=oracle.token_inputs(inp)):
        got[r0:r1] = out
        seen[r0:r1] = True
    assert seen.all()
    grp = (np.searchsorted(offsets, np.arange(R), side="right") - 1).astype(np.int32)
    if cfg.dispatch == "fp8":
        q, qp = oracle.fp8_quantize(inp.x[src[:R]])
        rows = oracle.fp8_dequantize(q, qp)
    else:
        rows = oracle.rows_as_f64(inp.x[src[:R]])
    ref = oracle.expert_rows(rows, grp, inp.w1, inp.w3, inp.w2, nthreads=4)
    assert _rel(got, ref) <= REL
    toks = np.arange(0, cfg.T, 5)
    sh = oracle.shared_rows(inp, toks)
    ref_sh = np.zeros_like(sh)
    for s in range(cfg.S):
        ref_sh += oracle.expert_rows(oracle.rows_as_f64(inp.x[toks]),
                                     np.full(len(toks), cfg.E + s, dtype=np.int32),
                                     inp.w1, inp.w3, inp.w2)
    assert _rel(sh, ref_sh) <= REL


def test_token_subset_equals_rows_of_the_whole_batch():
    cfg = _cfg("fp8_dispatch", T=200, d=64, h=32, E=6, k=3, S=1)
    inp = make_inputs(cfg, seed=8)
    idx, w, y = oracle.layer_dense(inp, chunk=33)
    toks = np.array([0, 5, 6, 77, 199])
    i2, w2, y2 = oracle.layer_dense(inp, tokens=toks, gate=(idx, w))
    assert np.array_equal(i2, idx[toks]) and np.array_equal(w2, w[toks])
    assert _rel(y2, y[toks]) <= REL


@pytest.mark.parametrize("name,kw", [
    ("deepseekmoe_bf16", dict(T=60, d=64, h=40, E=6, k=3, S=2)),
    ("fp8_dispatch", dict(T=50, d=48, h=24, E=5, k=2, S=1)),
    ("tiny_fp32", dict(T=40, d=16, h=12, E=4, k=2)),
])
def test_ffn_backward_matches_the_layer_backward(name, kw):
    """The expert stage's backward, fed the gradient that combine's backward
    hands it (w * dy for each kept slot's row, dy itself for the shared
    experts), gives the layer backward's expert weight gradients; and its row
    gradients, summed back per token (dispatch's backward) plus the gate's
    term, give the layer backward's dx."""
    cfg = dataclasses.replace(CONFIGS[name], sigma_w=0.2, **kw)
    inp = make_inputs(cfg, seed=11)
    T, k = cfg.T, cfg.k
    dy = np.random.default_rng(3).standard_normal((T, cfg.d))
    ref = oracle.layer_backward(inp, np.arange(T), dy)
    z = oracle.gate_logits(inp.x, inp.wg, inp.bias)
    idx, w = oracle.select_topk(z, k)
    counts, offsets, dest, src = oracle.dispatch(idx, cfg.E)
    dy_perm = np.zeros((int(offsets[-1]), cfg.d))
    for t in range(T):
        for j in range(k):
            dy_perm[dest[t, j]] = w[t, j] * dy[t]
    got = oracle.ffn_backward(inp, offsets, src, dy_perm, dy if cfg.S else None)
    for key in ("dw1", "dw3", "dw2"):
        assert _rel(got[key], ref[key]) <= 1e-11, key
    dx = np.zeros((T, cfg.d))
    for t in range(T):
        for j in range(k):
            dx[t] += got["dx_perm"][dest[t, j]]
    if cfg.S:
        dx += got["dx_shared"]
    _, dxg, _ = oracle.gate_backward(inp.x, inp.wg, idx, w, ref["dtopk_w"])
    assert _rel(dx + dxg, ref["dx"]) <= 1e-11
