"""GPU parity of the fp8 quantiser's per-expert and global modes (gsyq.cn
section 5.2: the same min/max affine map with the range taken over every row
dispatched to an expert, or over the whole batch) against the oracle.

Bars: the dispatch arrays bit-exact; every dispatched row's e4m3 codes and
(scale, centre) bit-exact against the oracle quantising that row from its
group's range (the min/max over the group's rows, taken with numpy); the layer
output within 6e-2 relative L2 against the oracle with per-slot ranges.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gpu_util import ORACLE_THREADS, RowErrors, dev, host, rel_l2, requires_gpu, say
from moe_workloads import CONFIGS, bf16_bits_to_f32, make_inputs

pytestmark = [pytest.mark.gpu, requires_gpu]


def _mm():
    import mixture_experts_routing_gemm_amd as mm
    return mm


def _cfg(**kw):
    base = dict(T=2000, d=512, E=16, k=4, S=1, h=128, sigma_w=0.05)
    base.update(kw)
    return dataclasses.replace(CONFIGS["fp8_dispatch"], name="fp8_modes", **base)


def group_ranges(xf, offsets, src, quant):
    """(min, max) per dispatched row: its own, its expert's rows' or the batch's."""
    n = int(offsets[-1])
    r = np.empty((n, 2), dtype=np.float32)
    if quant == "token":
        rows = xf[src[:n]]
        r[:, 0], r[:, 1] = rows.min(1), rows.max(1)
        return r
    if quant == "global":
        r[:] = (xf.min(), xf.max())
        return r
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            rows = xf[src[a:b]]
            r[a:b] = (rows.min(), rows.max())
    return r


def qrange_of(rr, dest):
    """(min, max) range [T,k,2] of each slot's row (zeros for a dropped slot)"""
    T, k = dest.shape
    q = np.zeros((T, k, 2), dtype=np.float32)
    kept = dest >= 0
    q[kept] = rr[dest[kept]]
    return q


def run_case(cfg, toks=None):
    mm = _mm()
    say(f"[fp8 modes] T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} S={cfg.S} quant={cfg.quant} "
        f"capacity={cfg.capacity} reassign={cfg.reassign}")
    inp = make_inputs(cfg, seed=3)
    shape = mm.shape_of(cfg)
    assert shape.quant == {"token": 0, "expert": 1, "global": 2}[cfg.quant]
    oidx, ow, _ = oracle.gate_topk(inp.x, inp.wg, cfg.k, inp.bias, nthreads=ORACLE_THREADS)
    counts, offsets, dest, src, route = oracle.dispatch(oidx, cfg.E, capacity=cfg.capacity,
                                                        reassign=cfg.reassign, return_route=True)
    n = int(offsets[cfg.E])
    xf = bf16_bits_to_f32(inp.x)
    rr = group_ranges(xf, offsets, src, cfg.quant)
    q_ref, qp_ref = oracle.fp8_quantize(inp.x[src[:n]], ranges=rr)

    # the dispatch stage alone, from the oracle's routing
    T, E, k, d = cfg.T, cfg.E, cfg.k, cfg.d
    g = dict(counts=torch.empty(E, dtype=torch.int32, device="cuda"),
             offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
             dest=torch.empty((T, k), dtype=torch.int32, device="cuda"),
             src=torch.empty(T * k, dtype=torch.int32, device="cuda"))
    x_perm = torch.empty((T * k, d), dtype=torch.uint8, device="cuda")
    qp = torch.empty((T * k, 2), dtype=torch.float32, device="cuda")
    ws = mm.alloc_workspace(shape, mm.STAGE_DISPATCH)
    mm.moe_dispatch(shape, dev(inp.x), dev(oidx), g["counts"], g["offsets"], g["dest"], g["src"],
                    x_perm, qp, ws)
    assert mm.moe_get_device_error(ws) == mm.MOE_OK
    assert np.array_equal(host(g["counts"]), counts)
    assert np.array_equal(host(g["offsets"]), offsets)
    assert np.array_equal(host(g["dest"]), dest)
    assert np.array_equal(host(g["src"])[:n], src[:n])
    assert np.array_equal(host(x_perm)[:n], q_ref), "fp8 codes differ"
    assert np.array_equal(host(qp)[:n].view(np.uint32), qp_ref.view(np.uint32))

    # the whole layer
    buf = mm.ForwardBuffers(shape)
    buf.run(dev(inp.x), dev(inp.wg), None if inp.bias is None else dev(inp.bias),
            dev(inp.w1), dev(inp.w3), dev(inp.w2))
    torch.cuda.synchronize()
    assert mm.moe_get_device_error(buf.ws) == mm.MOE_OK
    assert np.array_equal(host(buf.dest_row), dest)
    if toks is None:
        toks = np.arange(T)
    qrange_all = qrange_of(rr, dest)
    _, _, oy = oracle.layer_dense(inp, nthreads=ORACLE_THREADS, route=route, qrange=qrange_all,
                                  tokens=toks)
    acc = RowErrors()
    acc.add(host(buf.y)[toks], oy)
    acc.check(f"[fp8 modes] y on {len(toks)} tokens", cfg.tol_y)


@pytest.mark.parametrize("quant", ["expert", "global"])
def test_fp8_group_modes(quant):
    run_case(_cfg(quant=quant))


@pytest.mark.parametrize("quant", ["expert", "global"])
def test_fp8_group_modes_with_reassignment(quant):
    run_case(_cfg(quant=quant, T=1500, E=32, k=6, capacity=200, reassign=True))


def test_fp8_expert_mode_at_larger_size():
    cfg = _cfg(quant="expert", T=8192, d=1024, E=64, k=6, S=2, h=256)
    run_case(cfg, toks=np.array([0, 1, 17, 999, 4096, 8000, 8191], dtype=np.int64))


def test_token_mode_is_the_default_path():
    # quant = "token" must be the per-token kernel: same codes as before
    run_case(_cfg(quant="token", T=600))


def test_full_size_fp8_workload_per_expert_ranges():
    # fp8_dispatch at its full size with per-expert ranges, as bench.py
    # --quant expert times it: the dispatch arrays bit-exact, the codes and
    # (scale, centre) of sampled dispatched rows bit-exact, y on 4096 tokens
    mm = _mm()
    cfg = dataclasses.replace(CONFIGS["fp8_dispatch"], quant="expert")
    say(f"[fp8 modes] full size T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} quant=expert")
    inp = make_inputs(cfg)
    shape = mm.shape_of(cfg)
    oidx, ow, _ = oracle.gate_topk(inp.x, inp.wg, cfg.k, None, nthreads=ORACLE_THREADS)
    counts, offsets, dest, src = oracle.dispatch(oidx, cfg.E)
    n = int(offsets[cfg.E])
    xf = bf16_bits_to_f32(inp.x)
    rr = group_ranges(xf, offsets, src, "expert")
    T, E, k, d = cfg.T, cfg.E, cfg.k, cfg.d
    g_counts = torch.empty(E, dtype=torch.int32, device="cuda")
    g_offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    g_dest = torch.empty((T, k), dtype=torch.int32, device="cuda")
    g_src = torch.empty(T * k, dtype=torch.int32, device="cuda")
    x_perm = torch.empty((T * k, d), dtype=torch.uint8, device="cuda")
    qp = torch.empty((T * k, 2), dtype=torch.float32, device="cuda")
    ws = mm.alloc_workspace(shape, mm.STAGE_DISPATCH)
    xd = dev(inp.x)
    mm.moe_dispatch(shape, xd, dev(oidx), g_counts, g_offsets, g_dest, g_src, x_perm, qp, ws)
    assert mm.moe_get_device_error(ws) == mm.MOE_OK
    assert np.array_equal(host(g_counts), counts)
    assert np.array_equal(host(g_offsets), offsets)
    assert np.array_equal(host(g_dest), dest)
    assert np.array_equal(host(g_src)[:n], src[:n])
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([rng.integers(0, n, 3000), offsets[:-1][counts > 0],
                                     offsets[1:][counts > 0] - 1]))
    q_ref, qp_ref = oracle.fp8_quantize(inp.x[src[rows]], ranges=rr[rows])
    assert np.array_equal(host(x_perm)[rows], q_ref)
    assert np.array_equal(host(qp)[rows].view(np.uint32), qp_ref.view(np.uint32))
    del x_perm, qp, ws
    buf = mm.ForwardBuffers(shape)
    buf.run(xd, dev(inp.wg), None, dev(inp.w1), dev(inp.w3), dev(inp.w2))
    torch.cuda.synchronize()
    assert mm.moe_get_device_error(buf.ws) == mm.MOE_OK
    assert np.array_equal(host(buf.dest_row), dest)
    # y on 4096 tokens: a contiguous run, random ones and the ends
    rng = np.random.default_rng(3)
    toks = np.unique(np.concatenate([np.arange(1000, 3048), rng.integers(0, T, 2048),
                                     [0, 1, T - 1]])).astype(np.int64)
    _, _, oy = oracle.layer_dense(inp, nthreads=ORACLE_THREADS, qrange=qrange_of(rr, dest),
                                  tokens=toks, gate=(oidx, ow))
    acc = RowErrors()
    acc.add(host(buf.y)[toks], oy)
    acc.check(f"[fp8 modes] full size y on {len(toks)} tokens", cfg.tol_y)
