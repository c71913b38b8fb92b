"""GPU parity of the capacity-limited dispatch (a strict per-expert row cap;
assignments beyond it, in token order, are dropped or reassigned to the
least-loaded expert) against the oracle.

Bars as in the other parity tests: routing and every dispatch array
bit-exact, the dispatched rows a bit-exact copy, and the layer output within
the workload's relative-L2 bound (over the tensor and on every token) on
every token of the large cases and on chosen tokens of the others, where the oracle's
per-slot route comes from its own capacity dispatch over the whole batch.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gpu_util import ORACLE_THREADS, RowErrors, dev, host, requires_gpu, say
from moe_workloads import CONFIGS, make_inputs

pytestmark = [pytest.mark.gpu, requires_gpu]


def _mm():
    import mixture_experts_routing_gemm_amd as mm
    return mm


def forward_vs_oracle(inp, toks=None):
    mm, cfg = _mm(), inp.cfg
    say(f"[capacity] T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} S={cfg.S} h={cfg.h} "
        f"act={cfg.act} dispatch={cfg.dispatch} capacity={cfg.capacity} reassign={cfg.reassign}")
    shape = mm.shape_of(cfg)
    assert shape.capacity == cfg.capacity and shape.overflow == int(cfg.reassign)
    buf = mm.ForwardBuffers(shape)
    bias = None if inp.bias is None else dev(inp.bias)
    buf.run(dev(inp.x), dev(inp.wg), bias, dev(inp.w1), dev(inp.w3), dev(inp.w2))
    torch.cuda.synchronize()
    assert mm.moe_get_device_error(buf.ws) == mm.MOE_OK
    oidx, ow, _ = oracle.gate_topk(inp.x, inp.wg, cfg.k, inp.bias, nthreads=ORACLE_THREADS)
    counts, offsets, dest, src, route = oracle.dispatch(oidx, cfg.E, capacity=cfg.capacity,
                                                        reassign=cfg.reassign, return_route=True)
    n = int(offsets[cfg.E])
    say(f"[capacity] kept {n} of {cfg.T * cfg.k} assignments")
    assert np.array_equal(host(buf.topk_idx), oidx)
    assert np.array_equal(host(buf.counts), counts)
    assert np.array_equal(host(buf.offsets), offsets)
    assert np.array_equal(host(buf.dest_row), dest)
    assert np.array_equal(host(buf.src_token)[:n], src[:n])
    if toks is None:
        toks = np.arange(cfg.T)
    _, _, oy = oracle.layer_dense(inp, nthreads=ORACLE_THREADS, route=route, tokens=toks,
                                  gate=(oidx, ow))
    acc = RowErrors()
    acc.add(host(buf.y)[toks], oy)
    acc.check(f"[capacity] y on {len(toks)} tokens", cfg.tol_y)
    return buf, route


@pytest.mark.parametrize("name", ["zipf_capacity_bf16", "zipf_reassign_bf16"])
def test_skewed_workload_with_capacity(name):
    cfg = CONFIGS[name]
    inp = make_inputs(cfg)
    rng = np.random.default_rng(0)
    # the oracle's route decides which tokens lost or moved a slot; take some
    # of those, some that kept their experts, and the ends
    oidx, _, _ = oracle.gate_topk(inp.x, inp.wg, cfg.k, inp.bias, nthreads=ORACLE_THREADS)
    _, _, _, _, route = oracle.dispatch(oidx, cfg.E, capacity=cfg.capacity, reassign=cfg.reassign,
                                        return_route=True)
    moved = np.nonzero((route != oidx).any(axis=1))[0]
    same = np.nonzero((route == oidx).all(axis=1))[0]
    assert len(moved) > 0 and len(same) > 0
    toks = np.unique(np.concatenate([rng.choice(moved, 24), rng.choice(same, 16),
                                     [0, cfg.T - 1]])).astype(np.int64)
    buf, _ = forward_vs_oracle(inp, toks)
    if cfg.reassign and cfg.T * cfg.k == cfg.E * cfg.capacity:
        assert np.all(host(buf.counts) == cfg.capacity)  # every expert equally loaded


def test_capacity_dispatch_stage_payload():
    # moe_dispatch alone, from the oracle's routing: the kept rows are a copy
    mm = _mm()
    cfg = dataclasses.replace(CONFIGS["zipf_capacity_bf16"], T=3000, capacity=40)
    inp = make_inputs(cfg, seed=4)
    oidx, _, _ = oracle.gate_topk(inp.x, inp.wg, cfg.k, inp.bias, nthreads=ORACLE_THREADS)
    counts, offsets, dest, src = oracle.dispatch(oidx, cfg.E, capacity=cfg.capacity)
    n = int(offsets[cfg.E])
    T, E, k, d = cfg.T, cfg.E, cfg.k, cfg.d
    shape = mm.shape_of(cfg)
    g_counts = torch.empty(E, dtype=torch.int32, device="cuda")
    g_offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    g_dest = torch.empty((T, k), dtype=torch.int32, device="cuda")
    g_src = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    x = dev(inp.x)
    x_perm = torch.zeros((T * k, d), dtype=torch.bfloat16, device="cuda")
    ws = mm.alloc_workspace(shape, mm.STAGE_DISPATCH)
    mm.moe_dispatch(shape, x, dev(oidx), g_counts, g_offsets, g_dest, g_src, x_perm, None, ws)
    assert mm.moe_get_device_error(ws) == mm.MOE_OK
    assert np.array_equal(host(g_counts), counts)
    assert np.array_equal(host(g_offsets), offsets)
    assert np.array_equal(host(g_dest), dest)
    gs = host(g_src)
    assert np.array_equal(gs[:n], src[:n])
    assert np.all(gs[n:] == -7)  # nothing written past the kept rows
    sel = dev(src[:n].astype(np.int64))
    assert torch.equal(x_perm[:n].view(torch.int16), x[sel].view(torch.int16))
    assert int(torch.count_nonzero(x_perm[n:].view(torch.int16))) == 0


def _small(act="bf16", **kw):
    base = CONFIGS["tiny_fp32" if act == "f32" else "deepseekmoe_bf16"]
    kw.setdefault("sigma_w", 0.05)
    return dataclasses.replace(base, name="capacity_edge", **kw)


@pytest.mark.parametrize("kw", [
    dict(T=300, d=128, E=8, k=2, S=1, h=64, capacity=1),        # one row per expert
    dict(T=300, d=128, E=8, k=2, S=1, h=64, capacity=1, reassign=True),  # all but 8 dropped
    dict(T=520, d=256, E=16, k=4, S=0, h=128, capacity=90, reassign=True),  # some overflow left
    dict(T=512, d=128, E=16, k=2, S=0, h=64, capacity=64, reassign=True),   # exactly full
    dict(T=700, d=128, E=256, k=8, S=2, h=64, capacity=30, reassign=True),  # largest E and k
    dict(T=520, d=256, E=16, k=4, S=0, h=128, capacity=90),     # binds on some experts
    dict(T=400, d=128, E=8, k=2, S=0, h=64, capacity=400),      # never binds
    dict(T=600, d=256, E=32, k=8, S=2, h=128, capacity=100, dispatch="fp8", tol_y=6e-2),
    dict(T=600, d=256, E=32, k=8, S=2, h=128, capacity=160, dispatch="fp8", tol_y=6e-2,
         reassign=True),
], ids=["cap_1", "re_cap_1", "re_overflow_left", "re_exact", "re_max_E_k", "cap_binds",
        "cap_never_binds", "fp8_cap", "fp8_re"])
def test_bf16_capacity_shapes(kw):
    forward_vs_oracle(make_inputs(_small(**kw), seed=6))


@pytest.mark.parametrize("reassign", [False, True])
def test_f32_capacity_odd_dims(reassign):
    forward_vs_oracle(make_inputs(_small("f32", T=97, d=36, E=5, k=2, S=1, h=50, capacity=20,
                                         reassign=reassign, tol_y=1e-5), seed=7))


def test_capacity_never_binding_equals_dropless():
    mm = _mm()
    cfg = _small(T=500, d=128, E=8, k=2, S=1, h=64)
    inp = make_inputs(cfg, seed=8)
    outs = []
    for cap, re in ((0, False), (cfg.T, False), (cfg.T, True)):
        buf = mm.ForwardBuffers(mm.shape_of(dataclasses.replace(cfg, capacity=cap, reassign=re)))
        buf.run(dev(inp.x), dev(inp.wg), None, dev(inp.w1), dev(inp.w3), dev(inp.w2))
        torch.cuda.synchronize()
        outs.append((host(buf.y).copy(), host(buf.dest_row).copy()))
    for y, dest in outs[1:]:
        assert np.array_equal(outs[0][0], y) and np.array_equal(outs[0][1], dest)


def test_full_size_skewed_workload_reassigned_at_factor_1():
    # zipf_stress_bf16 at its full size, as bench.py --capacity-factor 1.0
    # --reassign times it: every dispatch array bit-exact, y on every token
    base = CONFIGS["zipf_stress_bf16"]
    cfg = dataclasses.replace(base, capacity=base.T * base.k // base.E, reassign=True)
    inp = make_inputs(cfg)
    buf, route = forward_vs_oracle(inp)
    assert np.all(host(buf.counts) == cfg.capacity)
