"""Checks of the synthetic workload recipe itself (not of the method)."""

import os

import numpy as np
import pytest

import oracle
from moe_workloads import CONFIGS, make_inputs, make_routing


def test_zipf_skew_hits_the_target_band():
    # the skewed workload must give expert 0 about 85-90 % of top-1 picks
    cfg = CONFIGS["zipf_stress_bf16"]
    inp = make_inputs(cfg, gate_only=True)
    idx, _, _ = oracle.gate_topk(inp.x[:4096], inp.wg, cfg.k, inp.bias, nthreads=os.cpu_count())
    share = np.mean(idx[:, 0] == 0)
    assert 0.85 <= share <= 0.90, share
    counts = np.bincount(idx.ravel(), minlength=cfg.E)
    assert (counts == 0).sum() > 50  # many experts receive nothing


def test_fp8_workload_has_outliers():
    cfg = CONFIGS["fp8_dispatch"]
    inp = make_inputs(cfg, T=512, gate_only=True)
    xf = (inp.x.astype(np.uint32) << 16).view(np.float32)
    frac = np.mean(np.abs(xf) > 8)
    assert 3e-4 < frac < 2e-3


def test_draws_are_reproducible():
    cfg = CONFIGS["tiny_fp32"]
    a, b = make_inputs(cfg), make_inputs(cfg)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.w2, b.w2)
    assert a.w1.std() == pytest.approx(1 / 8, rel=0.05)
    r = make_routing(100, 10, 3)
    assert all(len(set(row)) == 3 for row in r.tolist())
