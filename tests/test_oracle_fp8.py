"""Pins for the oracle's per-token affine FP8 (OCP e4m3) quantiser.

The e4m3 decoder and encoder are checked against torch's float8_e4m3fn CPU
casts; the per-row map against its defining properties (gsyq.cn section 3.1:
per token min/max, then an affine map): the endpoints land on +-448, a
constant row is reproduced exactly, and every element is within half an e4m3
step (times the scale) of its input.
"""

import numpy as np
import pytest
import torch

import oracle
from moe_workloads import to_bf16_bits

E4M3 = torch.float8_e4m3fn


def _torch_decode(code):
    return float(torch.tensor([code], dtype=torch.uint8).view(E4M3).float()[0])


def _torch_encode(v):
    return int(torch.tensor([v], dtype=torch.float32).to(E4M3).view(torch.uint8)[0])


def test_decode_all_codes_match_torch():
    for c in range(256):
        a, b = oracle.e4m3_decode(c), _torch_decode(c)
        if np.isnan(b):
            assert np.isnan(a)
        else:
            assert a == b, (c, a, b)
    assert oracle.e4m3_decode(0x7E) == 448.0 and oracle.e4m3_decode(0x01) == 2.0 ** -9


def test_encode_matches_torch_cast():
    rng = np.random.default_rng(0)
    reps = np.array([oracle.e4m3_decode(c) for c in range(0x7F)])
    mids = (reps[1:] + reps[:-1]) / 2          # exact ties
    vals = np.concatenate([
        reps, -reps, mids, -mids,
        np.nextafter(mids.astype(np.float32), np.float32(0)),
        np.nextafter(mids.astype(np.float32), np.float32(1000)),
        rng.uniform(-448, 448, 4000), rng.uniform(-0.03, 0.03, 2000),
        [0.0, -0.0, 1e-30, -1e-30, 2.0 ** -10, 2.0 ** -10 * 1.0001],
    ]).astype(np.float32)
    vals = vals[np.abs(vals) <= 448]
    ours = np.array([oracle.e4m3_encode(v) for v in vals])
    ref = torch.from_numpy(vals).to(E4M3).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, [(float(vals[i]), int(ours[i]), int(ref[i])) for i in bad[:5]]


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_row_map_properties(act):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    x[3, 17] *= 50  # an outlier
    xs = x if act == "f32" else to_bf16_bits(x)
    xf = x if act == "f32" else (xs.astype(np.uint32) << 16).view(np.float32)
    q, qp = oracle.fp8_quantize(xs)
    s, c = qp[:, 0].astype(np.float64), qp[:, 1].astype(np.float64)
    mn, mx = xf.min(axis=1).astype(np.float64), xf.max(axis=1).astype(np.float64)
    np.testing.assert_allclose(c, (mx + mn) / 2, rtol=1e-6)
    np.testing.assert_allclose(s, (mx - mn) / 2 / 448, rtol=1e-6)
    # endpoints land on the extreme codes
    t = np.arange(64)
    assert np.all(q[t, xf.argmax(axis=1)] == 0x7E)
    assert np.all(q[t, xf.argmin(axis=1)] == 0xFE)
    # per-element error bound: half an e4m3 step at |v|, times s, plus fp32 slop
    dq = oracle.fp8_dequantize(q, qp)
    v = np.abs((xf.astype(np.float64) - c[:, None]) / s[:, None])
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
    half_step = 2.0 ** (e - 3) / 2
    err = np.abs(dq - xf)
    assert np.all(err <= s[:, None] * half_step * (1 + 1e-5) + 1e-6 * np.abs(xf))


def test_constant_row_is_exact():
    x = np.full((3, 64), 1.25, dtype=np.float32)
    x[1] = -3.5
    x[2] = 0.0
    q, qp = oracle.fp8_quantize(x)
    assert np.all(q == 0) and np.all(qp[:, 0] == 0)
    assert np.array_equal(oracle.fp8_dequantize(q, qp), x.astype(np.float64))


# ------------------------------------------- per-expert / global ranges ----
# The quantiser's other modes (gsyq.cn section 5.2: per-token, per-expert,
# global) map a row from a range wider than its own min/max: the expert's
# rows' or the whole batch's. Pinned by the per-token map (a row's own range
# must give the same codes) and by torch's e4m3 cast of the affine map
# written out in float32.

def _f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_own_range_equals_per_token_map():
    rng = np.random.default_rng(3)
    x = to_bf16_bits(rng.standard_normal((40, 96)).astype(np.float32) * 3)
    q, qp = oracle.fp8_quantize(x)
    xf = _f32(x)
    q2, qp2 = oracle.fp8_quantize(x, ranges=np.stack([xf.min(1), xf.max(1)], 1))
    assert np.array_equal(q, q2) and np.array_equal(qp.view(np.uint32), qp2.view(np.uint32))


def test_wider_range_matches_torch_cast():
    rng = np.random.default_rng(4)
    x = to_bf16_bits(rng.standard_normal((64, 128)).astype(np.float32))
    xf = _f32(x)
    mn, mx = np.float32(xf.min() - 1.5), np.float32(xf.max() + 0.25)   # a group's wider range
    ranges = np.tile(np.array([mn, mx], dtype=np.float32), (64, 1))
    q, qp = oracle.fp8_quantize(x, ranges=ranges)
    c = np.float32(0.5) * (mx + mn)
    r = np.float32(0.5) * (mx - mn)
    inv = np.float32(448.0) / r
    v = np.clip((xf - c) * inv, -448.0, 448.0).astype(np.float32)
    ref = torch.from_numpy(v).to(E4M3).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)
    assert np.all(qp[:, 0] == r / np.float32(448.0)) and np.all(qp[:, 1] == c)
    # the range's ends, where a row reaches them, land on the ends of e4m3
    x2 = x.copy()
    x2[0, 0], x2[0, 1] = to_bf16_bits(np.array([-3.0, 5.0], dtype=np.float32))
    q2, _ = oracle.fp8_quantize(x2, ranges=np.tile(np.array([-3.0, 5.0], np.float32), (64, 1)))
    assert oracle.e4m3_decode(int(q2[0, 0])) == -448.0 and oracle.e4m3_decode(int(q2[0, 1])) == 448.0


def test_range_must_be_ordered():
    x = to_bf16_bits(np.ones((1, 16), dtype=np.float32))
    with pytest.raises(ValueError):
        oracle.fp8_quantize(x, ranges=np.array([[1.0, 0.5]], dtype=np.float32))
