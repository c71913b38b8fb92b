"""Pins for the oracle's fp8-weight variant and the symmetric absmax mode.

The pages define FP8 only for the dispatched activations; the oracle's
reading for weights (and the hidden rows) is a symmetric absmax e4m3 scale
per row: the activations' affine map over [-max|w|, max|w|]. Pinned by
torch's own float8_e4m3fn cast (a library encoder, not the oracle's): codes
of rows, exact round trips of representable rows, and the whole fp8-weight
layer recomputed with torch casts and float64 torch matmuls.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from moe_workloads import CONFIGS, bf16_bits_to_f32, make_inputs


def torch_codes(rows32):
    """symmetric absmax e4m3 codes by torch's cast of the written-out map"""
    r = torch.from_numpy(rows32)
    amax = r.abs().amax(dim=1, keepdim=True)
    inv = torch.where(amax > 0, torch.tensor(448.0) / amax, torch.zeros_like(amax))
    v = torch.clamp(r * inv, -448.0, 448.0)
    q = v.to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy(), (amax / 448.0).squeeze(1).numpy()


def test_weight_rows_match_torch_cast():
    rng = np.random.default_rng(0)
    w = (rng.standard_normal((3, 40, 64), dtype=np.float32) * 0.02)
    w[1, 5] = 0.0                      # an all-zero row
    w[2, 7, 3] = 1.5                   # an outlier
    q, s = oracle.quantize_weight_rows(w)
    tq, ts = torch_codes(w.reshape(-1, 64))
    assert np.array_equal(q.reshape(-1, 64), tq)
    assert np.array_equal(s.reshape(-1), ts.astype(np.float32))
    assert np.all(q[1, 5] == 0) and s[1, 5] == 0.0
    # the largest magnitude maps to +-448 (code 0x7e / 0xfe)
    i = np.argmax(np.abs(w[2, 7]))
    assert q[2, 7, i] & 0x7F == 0x7E


def test_representable_rows_round_trip_exactly():
    # a row made of e4m3 values times a power-of-two scale, with one element
    # at +-448 of it, quantises to itself
    vals = np.array([448.0, -448.0, 1.0, -2.5, 0.0, 0.125, 96.0, -0.015625], dtype=np.float32)
    rng = np.random.default_rng(1)
    rows = np.stack([rng.permutation(vals) for _ in range(10)]) * np.float32(2.0 ** -10)
    q, s = oracle.quantize_weight_rows(rows)
    back = oracle.fp8_dequantize(q, np.stack([s, np.zeros_like(s)], axis=1))
    assert np.array_equal(back, rows.astype(np.float64))


def test_token_absmax_rows_are_centred():
    cfg = dataclasses.replace(CONFIGS["fp8_dispatch"], T=50, d=64, h=32, E=4, k=2, S=1,
                              quant="token_absmax")
    inp = make_inputs(cfg, seed=2)
    x32 = bf16_bits_to_f32(inp.x)
    xq = oracle.token_inputs(inp)
    tq, ts = torch_codes(x32)
    ref = torch.from_numpy(tq).view(torch.float8_e4m3fn).to(torch.float64).numpy() * ts[:, None]
    assert np.array_equal(xq, ref)


def torch_layer_fp8w(inp):
    """The fp8-weight layer with torch casts for every quantisation step and
    float64 torch matmuls."""
    cfg = inp.cfg
    E, S, k, h = cfg.E, cfg.S, cfg.k, cfg.h
    x32 = bf16_bits_to_f32(inp.x)
    z = oracle.gate_logits(inp.x, inp.wg, inp.bias)
    idx, w = oracle.select_topk(z, k)
    # per-token affine fp8 rows (torch cast of the written-out map)
    xt = torch.from_numpy(x32)
    mn, mx = xt.amin(1, keepdim=True), xt.amax(1, keepdim=True)
    c = 0.5 * (mx + mn)
    r = 0.5 * (mx - mn)
    inv = torch.where(r > 0, torch.tensor(448.0) / r, torch.zeros_like(r))
    qx = torch.clamp((xt - c) * inv, -448.0, 448.0).to(torch.float8_e4m3fn).to(torch.float64)
    v = qx * (r / 448.0).double() + c.double()

    def deq(wrows):
        q, s = torch_codes(bf16_bits_to_f32(wrows))
        return torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64) * \
            torch.from_numpy(s).double()[:, None]

    def qh(hid):
        h32 = hid.float().to(torch.bfloat16).float().numpy()
        q, s = torch_codes(h32)
        return torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64) * \
            torch.from_numpy(s).double()[:, None]

    def hidden(vv, g):
        a = vv @ deq(inp.w1[g]).T
        b = vv @ deq(inp.w3[g]).T
        return a * torch.sigmoid(a) * b

    y = torch.zeros((cfg.T, cfg.d), dtype=torch.float64)
    if S:
        hq = qh(torch.cat([hidden(v, E + s) for s in range(S)], dim=1))
        # the shared W2 rows quantised jointly over the S blocks
        w2s = deq(np.concatenate([inp.w2[E + s] for s in range(S)], axis=1))
        y += hq @ w2s.T
    for t in range(cfg.T):
        for j in range(k):
            e = int(idx[t, j])
            hq = qh(hidden(v[t:t + 1], e))
            y[t] += float(w[t, j]) * (hq @ deq(inp.w2[e]).T)[0]
    return idx, y.numpy()


@pytest.mark.parametrize("kw", [dict(T=40, d=64, h=32, E=5, k=2, S=2),
                                dict(T=30, d=48, h=24, E=3, k=3, S=0)])
def test_fp8_weight_layer_matches_torch(kw):
    cfg = dataclasses.replace(CONFIGS["fp8_dispatch"], sigma_w=0.1, **kw)
    inp = make_inputs(cfg, seed=3)
    idx_t, y_t = torch_layer_fp8w(inp)
    idx, _, y = oracle.layer_dense_fp8w(inp, oracle.quantize_expert_weights(inp))
    assert np.array_equal(idx, idx_t)
    assert np.linalg.norm(y - y_t) / np.linalg.norm(y_t) <= 1e-12
