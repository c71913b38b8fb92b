"""Pins for the oracle's layer backward (gradients of sum(dy * y)).

Checked against (1) autograd of a float64 torch re-implementation of the
layer -- torch's autograd, a library routine, differentiates the forward
written out with the same readings (top-k choice fixed, fp8 rows straight
through, dropped slots kept in the softmax) -- and (2) central finite
differences of the oracle's own forward (layer_tokens), which shares no code
with the backward. The oracle's gate weights come from float32 logits, the
re-implementation's from float64 ones, hence the 1e-6 tolerances.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from moe_workloads import CONFIGS, bf16_bits_to_f32, make_inputs


def _f64(a):
    return torch.from_numpy(a.astype(np.float64) if a.dtype == np.float32
                            else bf16_bits_to_f32(a).astype(np.float64))


def _cfg(act="f32", **kw):
    base = CONFIGS["tiny_fp32" if act == "f32" else "deepseekmoe_bf16"]
    kw.setdefault("sigma_w", 0.3)
    return dataclasses.replace(base, **kw)


def torch_grads(inp, idx, dy, route=None):
    """Autograd of sum(dy * y) for the layer written out in float64 torch."""
    cfg = inp.cfg
    X = _f64(inp.x).requires_grad_(True)
    Wg = _f64(inp.wg).requires_grad_(True)
    W1 = _f64(inp.w1).requires_grad_(True)
    W3 = _f64(inp.w3).requires_grad_(True)
    W2 = _f64(inp.w2).requires_grad_(True)
    z = X @ Wg.T
    if inp.bias is not None:
        z = z + torch.from_numpy(inp.bias.astype(np.float64))
    I = torch.from_numpy(idx.astype(np.int64))
    w = torch.softmax(z.gather(1, I), dim=1)
    w.retain_grad()
    if cfg.dispatch == "fp8":
        q, qp = oracle.fp8_quantize(inp.x)
        Xq = X + (torch.from_numpy(oracle.fp8_dequantize(q, qp)) - X).detach()
    else:
        Xq = X

    def ffn(v, g):
        a = v @ W1[g].T
        return (a * torch.sigmoid(a) * (v @ W3[g].T)) @ W2[g].T

    y = torch.zeros_like(X)
    for s in range(cfg.S):
        y = y + ffn(X, cfg.E + s)
    for t in range(cfg.T):
        for j in range(cfg.k):
            e = int(idx[t, j]) if route is None else int(route[t, j])
            if e < 0:
                continue
            y[t] = y[t] + w[t, j] * ffn(Xq[t:t + 1], e)[0]
    (torch.from_numpy(dy) * y).sum().backward()
    return dict(dx=X.grad.numpy(), dwg=Wg.grad.numpy(), dw1=W1.grad.numpy(), dw3=W3.grad.numpy(),
                dw2=W2.grad.numpy(), dtopk_w=w.grad.numpy())


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("act,kw", [
    ("f32", dict(T=12, d=16, E=5, k=2, S=0, h=8)),
    ("f32", dict(T=9, d=12, E=4, k=4, S=2, h=10)),      # k = E, shared experts
    ("bf16", dict(T=10, d=16, E=6, k=3, S=1, h=8)),
    ("bf16", dict(T=8, d=16, E=6, k=2, S=1, h=8, dispatch="fp8")),
], ids=["f32", "k_eq_E_shared", "bf16", "fp8_rows"])
def test_backward_matches_autograd(act, kw):
    inp = make_inputs(_cfg(act, **kw), seed=3)
    cfg = inp.cfg
    toks = np.arange(cfg.T)
    idx, _, _ = oracle.layer_tokens(inp, toks)
    dy = np.random.default_rng(5).standard_normal((cfg.T, cfg.d))
    got = oracle.layer_backward(inp, toks, dy)
    ref = torch_grads(inp, idx, dy)
    for key in ("dx", "dwg", "dw1", "dw3", "dw2", "dtopk_w"):
        assert _rel(got[key], ref[key]) < 1e-6, (key, _rel(got[key], ref[key]))


def test_dropped_slot_has_no_output_gradient():
    inp = make_inputs(_cfg("f32", T=10, d=12, E=5, k=2, S=1, h=6), seed=4)
    cfg = inp.cfg
    toks = np.arange(cfg.T)
    idx, _, _ = oracle.layer_tokens(inp, toks)
    route = idx.copy()
    route[::2, 1] = -1
    dy = np.random.default_rng(6).standard_normal((cfg.T, cfg.d))
    got = oracle.layer_backward(inp, toks, dy, route=route)
    ref = torch_grads(inp, idx, dy, route=route)
    for key in ("dx", "dwg", "dw1", "dw3", "dw2", "dtopk_w"):
        assert _rel(got[key], ref[key]) < 1e-6, key
    assert np.all(got["dtopk_w"][::2, 1] == 0.0)


def test_backward_matches_finite_differences():
    inp = make_inputs(_cfg("f32", T=6, d=10, E=4, k=2, S=1, h=7), seed=7)
    cfg = inp.cfg
    toks = np.arange(cfg.T)
    dy = np.random.default_rng(8).standard_normal((cfg.T, cfg.d))
    idx0, _, _ = oracle.layer_tokens(inp, toks)
    g = oracle.layer_backward(inp, toks, dy)

    def loss():
        idx, _, y = oracle.layer_tokens(inp, toks)
        return float(np.sum(dy * y)), np.array_equal(idx, idx0)

    rng = np.random.default_rng(9)
    checks = [("w1", "dw1"), ("w3", "dw3"), ("w2", "dw2"), ("x", "dx"), ("wg", "dwg")]
    for arr_name, grad_name in checks:
        arr = getattr(inp, arr_name)
        done = 0
        for _ in range(40):
            if done == 4:
                break
            pos = tuple(rng.integers(0, s) for s in arr.shape)
            old = arr[pos]
            eps = np.float32(3e-3 if arr_name in ("x", "wg") else 1e-3)
            arr[pos] = old + eps
            hi_v, (lp, same_p) = arr[pos], loss()
            arr[pos] = old - eps
            lo_v, (lm, same_m) = arr[pos], loss()
            arr[pos] = old
            if not (same_p and same_m):
                continue  # the step crossed a routing boundary: not differentiable there
            fd = (lp - lm) / (float(hi_v) - float(lo_v))
            an = g[grad_name][pos]
            # the gate runs in float32, so its steps carry float32 noise
            tol = 2e-3 * max(1.0, abs(an)) if arr_name in ("x", "wg") else 1e-5 * max(1.0, abs(an))
            assert abs(fd - an) < tol, (arr_name, pos, fd, an)
            done += 1
        assert done == 4, arr_name


# ------------------------------------------- combine / dispatch backward ---
# Each is the transpose of a forward step the oracle already has, so the
# adjoint identity <forward(a), b> = <a, backward(b)> pins it; dtopk_w is
# also checked against the layer backward on the experts' real outputs.

def _rows_f32(rng, n, d):
    return rng.standard_normal((n, d)).astype(np.float32)


@pytest.mark.parametrize("capacity", [0, 25])
def test_combine_backward_is_the_transpose_of_combine(capacity):
    from moe_workloads import make_routing
    rng = np.random.default_rng(1)
    T, E, k, d = 200, 8, 3, 24
    idx = make_routing(T, E, k, seed=2, skew=1.0)
    _, offsets, dest, _ = oracle.dispatch(idx, E, capacity=capacity)
    w = rng.random((T, k)).astype(np.float32)
    Y = _rows_f32(rng, T * k, d)
    dy = _rows_f32(rng, T, d)
    y = oracle.combine(Y, None, np.where(dest >= 0, dest, 0), w * (dest >= 0))
    dyp, dw = oracle.combine_backward(dy, Y, dest, w)
    lhs = float(np.sum(y * dy.astype(np.float64)))
    rhs = float(np.sum(dyp * Y.astype(np.float64)))
    assert abs(lhs - rhs) <= 1e-9 * max(1.0, abs(lhs))
    # d w is the dot product of dy with the slot's row; dropped slots give 0
    kept = dest >= 0
    ref = np.einsum("td,tkd->tk", dy.astype(np.float64), Y[np.where(kept, dest, 0)].astype(np.float64))
    np.testing.assert_allclose(dw[kept], ref[kept], rtol=1e-12, atol=1e-12)
    assert np.all(dw[~kept] == 0.0)


def test_dispatch_backward_is_the_transpose_of_the_permutation():
    from moe_workloads import make_routing
    rng = np.random.default_rng(3)
    T, E, k, d = 150, 6, 2, 20
    idx = make_routing(T, E, k, seed=4)
    _, offsets, dest, src = oracle.dispatch(idx, E)
    x = _rows_f32(rng, T, d)
    g = _rows_f32(rng, T * k, d)
    sh = _rows_f32(rng, T, d)
    dx = oracle.dispatch_backward(g, sh, dest)
    lhs = float(np.sum(x[src].astype(np.float64) * g)) + float(np.sum(x.astype(np.float64) * sh))
    rhs = float(np.sum(x.astype(np.float64) * dx))
    assert abs(lhs - rhs) <= 1e-9 * max(1.0, abs(lhs))


def test_combine_backward_weights_match_the_layer_backward():
    inp = make_inputs(_cfg("f32", T=10, d=12, E=5, k=2, S=0, h=8), seed=5)
    cfg = inp.cfg
    toks = np.arange(cfg.T)
    idx, w, _ = oracle.layer_tokens(inp, toks)
    _, offsets, dest, src = oracle.dispatch(idx, cfg.E)
    groups = (np.searchsorted(offsets, np.arange(cfg.T * cfg.k), side="right") - 1).astype(np.int32)
    Y = oracle.expert_rows(oracle.rows_as_f64(inp.x[src]), groups, inp.w1, inp.w3, inp.w2)
    dy = np.random.default_rng(6).standard_normal((cfg.T, cfg.d)).astype(np.float32)
    _, dw = oracle.combine_backward(dy, Y.astype(np.float32), dest, w.astype(np.float32))
    ref = oracle.layer_backward(inp, toks, dy.astype(np.float64))["dtopk_w"]
    assert _rel(dw, ref) < 1e-6


def test_gate_backward_weight_gradient_matches_the_layer_backward():
    inp = make_inputs(_cfg("f32", T=10, d=12, E=5, k=2, S=0, h=8), seed=7)
    cfg = inp.cfg
    toks = np.arange(cfg.T)
    idx, w, _ = oracle.layer_tokens(inp, toks)
    dy = np.random.default_rng(8).standard_normal((cfg.T, cfg.d))
    ref = oracle.layer_backward(inp, toks, dy)
    _, _, dwg = oracle.gate_backward(inp.x, inp.wg, idx, w, ref["dtopk_w"])
    assert _rel(dwg, ref["dwg"]) < 1e-12


def _renormalised_topk(z, idx):
    """The renormalised top-k weights from the full softmax (its definition)."""
    p = np.exp(z - z.max())
    p /= p.sum()
    sel = p[idx]
    return sel / sel.sum()


def test_gate_logit_gradient_matches_finite_differences():
    """dz against central differences of f(z) = sum_j dw_j w_j(z), where w(z)
    is the full softmax restricted to the chosen experts and renormalised;
    the logits of unchosen experts must get exactly zero gradient."""
    rng = np.random.default_rng(9)
    E, k, d = 7, 3, 4
    z = rng.standard_normal(E)
    idx = np.argsort(-z, kind="stable")[:k].astype(np.int32)
    w = _renormalised_topk(z, idx)
    dw = rng.standard_normal(k)
    x = rng.standard_normal((1, d)).astype(np.float32)
    wg = rng.standard_normal((E, d)).astype(np.float32)
    dz, _, _ = oracle.gate_backward(x, wg, idx[None, :], w[None, :], dw[None, :])
    eps = 1e-6
    for e in range(E):
        zp, zm = z.copy(), z.copy()
        zp[e] += eps
        zm[e] -= eps
        fd = (dw @ _renormalised_topk(zp, idx) - dw @ _renormalised_topk(zm, idx)) / (2 * eps)
        pos = np.nonzero(idx == e)[0]
        got = dz[0, pos[0]] if pos.size else 0.0
        assert abs(got - fd) < 1e-8, (e, got, fd)
    assert abs(dz.sum()) < 1e-14


def test_gate_backward_top1_has_no_logit_gradient():
    """With k = 1 the weight is identically one."""
    rng = np.random.default_rng(10)
    x = rng.standard_normal((5, 8)).astype(np.float32)
    wg = rng.standard_normal((4, 8)).astype(np.float32)
    idx = rng.integers(0, 4, (5, 1)).astype(np.int32)
    dz, dxg, dwg = oracle.gate_backward(x, wg, idx, np.ones((5, 1)), rng.standard_normal((5, 1)))
    assert np.all(dz == 0.0) and np.all(dxg == 0.0) and np.all(dwg == 0.0)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_gate_backward_is_the_gate_gemm_transposed(act):
    """With dz scattered into a dense [T,E] matrix D: dx_gate = D Wg and
    dwg = D^T x (the two products of z = x Wg^T, by a library matmul)."""
    rng = np.random.default_rng(11)
    T, d, E, k = 37, 24, 9, 3
    x32 = rng.standard_normal((T, d)).astype(np.float32)
    wg32 = rng.standard_normal((E, d)).astype(np.float32)
    if act == "bf16":
        from moe_workloads import to_bf16_bits
        x, wg = to_bf16_bits(x32), to_bf16_bits(wg32)
        xf, wgf = bf16_bits_to_f32(x).astype(np.float64), bf16_bits_to_f32(wg).astype(np.float64)
    else:
        x, wg, xf, wgf = x32, wg32, x32.astype(np.float64), wg32.astype(np.float64)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)) + 0.1
    w /= w.sum(axis=1, keepdims=True)
    dw = rng.standard_normal((T, k))
    dz, dxg, dwg = oracle.gate_backward(x, wg, idx, w, dw)
    D = np.zeros((T, E))
    for t in range(T):
        D[t, idx[t]] = dz[t]
    assert _rel(dxg, D @ wgf) < 1e-13
    assert _rel(dwg, D.T @ xf) < 1e-13
