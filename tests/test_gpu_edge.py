"""GPU edge cases against the oracle at sizes it finishes in seconds: ragged
token counts, a single token, one expert, k = E, the largest E and k, empty
experts, constant rows on the fp8 path, bf16 / fp8 / float32 shapes off the
tile grid (any d % 8 == 0 -- 16 for fp8 rows -- and any h), bad
routing ids (turned into an error by the kernels' own checks), and T = 0."""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gpu_util import ORACLE_THREADS, RowErrors, act_torch, dev, host, rel_l2, requires_gpu, say
from moe_workloads import CONFIGS, make_inputs, make_routing

pytestmark = [pytest.mark.gpu, requires_gpu]


def _mm():
    import mixture_experts_routing_gemm_amd as mm
    return mm


def small_cfg(act="bf16", **kw):
    base = CONFIGS["tiny_fp32" if act == "f32" else "deepseekmoe_bf16"]
    kw.setdefault("sigma_w", 0.05)
    return dataclasses.replace(base, name="edge", **kw)


def forward_vs_oracle(inp):
    mm, cfg = _mm(), inp.cfg
    say(f"[edge] T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} S={cfg.S} h={cfg.h} act={cfg.act} "
        f"dispatch={cfg.dispatch}")
    shape = mm.shape_of(cfg)
    buf = mm.ForwardBuffers(shape)
    bias = None if inp.bias is None else dev(inp.bias)
    buf.run(dev(inp.x), dev(inp.wg), bias, dev(inp.w1), dev(inp.w3), dev(inp.w2))
    torch.cuda.synchronize()
    assert mm.moe_get_device_error(buf.ws) == mm.MOE_OK
    toks = np.arange(cfg.T)
    oidx, ow, oy = oracle.layer_tokens(inp, toks, nthreads=ORACLE_THREADS)
    counts, offsets, dest, src = oracle.dispatch(oidx, cfg.E)
    assert np.array_equal(host(buf.topk_idx), oidx)
    assert rel_l2(host(buf.topk_w), ow) <= 1e-5
    assert np.array_equal(host(buf.counts), counts)
    assert np.array_equal(host(buf.offsets), offsets)
    assert np.array_equal(host(buf.dest_row), dest)
    assert np.array_equal(host(buf.src_token)[: cfg.T * cfg.k], src)
    acc = RowErrors()
    acc.add(host(buf.y), oy)
    acc.check("[edge] y", cfg.tol_y)
    return buf, oidx


@pytest.mark.parametrize("kw", [
    dict(T=300, d=128, E=8, k=2, S=1, h=64),      # ragged T, partial tiles
    dict(T=1, d=256, E=8, k=3, S=2, h=128),       # a single token
    dict(T=257, d=128, E=1, k=1, S=0, h=64),      # one expert, one slot
    dict(T=200, d=128, E=4, k=4, S=0, h=192),     # k = E
    dict(T=700, d=128, E=256, k=8, S=2, h=64),    # largest E and k
    dict(T=520, d=384, E=16, k=2, S=0, h=320),    # several n tiles, ragged experts
], ids=["ragged", "one_token", "one_expert", "k_eq_E", "max_E_k", "wide"])
def test_bf16_shapes(kw):
    forward_vs_oracle(make_inputs(small_cfg(**kw), seed=1))


@pytest.mark.parametrize("kw", [
    dict(T=333, d=200, E=6, k=2, S=1, h=100),     # d % 128 != 0, h % 8 != 0
    dict(T=333, d=200, E=6, k=2, S=2, h=104),     # h % 64 != 0, shared blocks of 104
    dict(T=100, d=8, E=4, k=2, S=2, h=37),        # the narrowest rows, odd h
    dict(T=500, d=272, E=8, k=3, S=2, h=96, dispatch="fp8", tol_y=6e-2),   # fp8 rows, d % 256 != 0
    dict(T=64, d=16, E=3, k=1, S=1, h=5, dispatch="fp8", tol_y=6e-2),      # fp8, tiny h
], ids=["d200_h100", "d200_h104", "d8_h37", "fp8_d272_h96", "fp8_d16_h5"])
def test_bf16_shapes_off_the_tile_grid(kw):
    forward_vs_oracle(make_inputs(small_cfg(**kw), seed=5))


def test_grouped_ffn_stage_off_the_tile_grid():
    # moe_grouped_ffn alone on rows the oracle dispatched: every routed row
    # and every shared-expert sum
    mm = _mm()
    cfg = small_cfg(T=400, d=136, E=5, k=2, S=2, h=60)
    inp = make_inputs(cfg, seed=6)
    oidx, _, _ = oracle.gate_topk(inp.x, inp.wg, cfg.k, None)
    counts, offsets, dest, src = oracle.dispatch(oidx, cfg.E)
    shape = mm.shape_of(cfg)
    x = dev(inp.x)
    x_perm = x[dev(src.astype(np.int64))].contiguous()
    y_perm = torch.empty((cfg.T * cfg.k, cfg.d), dtype=torch.bfloat16, device="cuda")
    y_sh = torch.empty((cfg.T, cfg.d), dtype=torch.bfloat16, device="cuda")
    ws = mm.alloc_workspace(shape, mm.STAGE_FFN)
    mm.moe_grouped_ffn(shape, x_perm, None, dev(offsets), x, dev(inp.w1), dev(inp.w3),
                       dev(inp.w2), y_perm, y_sh, ws)
    torch.cuda.synchronize()
    got = host(y_perm)
    acc = RowErrors()
    for r0, r1, ref in oracle.routed_rows(inp, offsets, src):
        acc.add(got[r0:r1], ref, r0)
    acc.check("[edge] routed rows d=136 h=60", cfg.tol_y)
    acc = RowErrors()
    acc.add(host(y_sh), oracle.shared_rows(inp, np.arange(cfg.T)))
    acc.check("[edge] shared rows d=136 h=60", cfg.tol_y)


@pytest.mark.parametrize("kw", [
    dict(T=37, d=36, E=5, k=2, S=1, h=50),
    dict(T=130, d=64, E=8, k=2, S=0, h=128),
], ids=["odd_dims", "tiny_like"])
def test_f32_shapes(kw):
    forward_vs_oracle(make_inputs(small_cfg("f32", tol_y=1e-5, **kw), seed=2))


def test_empty_experts_and_a_hot_expert():
    cfg = small_cfg(T=1000, d=128, E=32, k=2, S=0, h=64)
    inp = make_inputs(cfg, seed=3)
    b = np.full(cfg.E, -50.0, dtype=np.float32)
    b[[0, 5, 9]] = [40.0, 20.0, 20.0]
    inp.bias = b
    buf, oidx = forward_vs_oracle(inp)
    counts = host(buf.counts)
    assert counts[0] == cfg.T and (counts == 0).sum() >= 29


def test_fp8_constant_rows_and_outliers():
    cfg = small_cfg(T=260, d=256, E=8, k=3, S=1, h=128, dispatch="fp8", outlier_p=0.01,
                    outlier_scale=50.0, tol_y=6e-2)
    inp = make_inputs(cfg, seed=4)
    inp.x[7] = inp.x[7, 0]      # constant row -> scale 0, codes 0
    inp.x[100] = 0              # zero row
    forward_vs_oracle(inp)


@pytest.mark.parametrize("act,T,d,E,k,bias", [
    ("bf16", 150, 200, 24, 3, True),      # K tail past the last 64-wide block
    ("bf16", 1000, 8, 3, 2, False),       # K shorter than one block
    ("f32", 77, 100, 9, 4, True),         # float32 weights, K tail
    ("bf16", 4100, 1096, 40, 5, False),   # partial last chunk, ragged token group
    ("bf16", 16384, 192, 16, 2, True),    # 64 tokens x 4 experts per lane
    ("bf16", 65536, 64, 64, 6, False),    # 32 tokens x 8 experts per lane
    ("bf16", 3000, 512, 50, 4, True),     # 16 tokens x 4 experts per lane
    ("f32", 500, 192, 100, 8, False),     # 16 tokens x 8 experts per lane, float32
    ("bf16", 300, 256, 200, 8, True),     # more experts than a block covers
    ("bf16", 513, 320, 256, 8, False),    # the most experts, ragged token block
    ("bf16", 129, 4096, 128, 1, True),    # k = 1, long chains
    ("bf16", 32845, 136, 128, 4, True),   # the size the two-phase gate takes by itself
], ids=["tail", "short_k", "f32", "partial_chunk", "tw64", "tw32", "tw16_me4", "f32_me8",
        "e200", "e256", "k1", "large"])
@pytest.mark.parametrize("path", ["auto", "two_phase", "one_phase"])
def test_gate_both_paths(act, T, d, E, k, bias, path, monkeypatch):
    """moe_gate_topk with a logits buffer (every logit's chain, then the
    top-k) and without (bf16: approximate logits on the matrix cores and
    exact chains for the candidates only): bit-exact logits and ids in both,
    the same weight bits in both, weights to 1e-5 of the oracle's."""
    mm = _mm()
    cfg = small_cfg(act, T=T, d=d, E=E, k=k, S=0, h=64, tol_y=1e-5)
    inp = make_inputs(cfg, seed=11, gate_only=True)
    if bias:
        inp.bias = np.random.default_rng(12).normal(0.0, 0.05, E).astype(np.float32)
    monkeypatch.setenv("MOE_GATE_PATH", path)
    say(f"[gate] act={act} T={T} d={d} E={E} k={k} bias={bias} path={path}")
    z_ref = oracle.gate_logits(inp.x, inp.wg, inp.bias, nthreads=ORACLE_THREADS)
    idx_ref, w_ref = oracle.select_topk(z_ref, k)
    shape = mm.shape_of(cfg)
    x, wg = dev(inp.x), dev(inp.wg)
    b = None if inp.bias is None else dev(inp.bias)
    ws_bits = []
    for with_logits in (True, False):
        idx = torch.full((T, k), -3, dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        z = torch.empty((T, E), dtype=torch.float32, device="cuda") if with_logits else None
        mm.moe_gate_topk(shape, x, wg, b, idx, w, z)
        torch.cuda.synchronize()
        if with_logits:
            nbad = int(np.sum(host(z).view(np.uint32) != z_ref.view(np.uint32)))
            assert nbad == 0, f"{nbad} logits differ"
        assert np.array_equal(host(idx), idx_ref), f"ids differ (logits buffer: {with_logits})"
        assert rel_l2(host(w), w_ref) <= 1e-5
        ws_bits.append(host(w).view(np.uint32).copy())
    assert np.array_equal(ws_bits[0], ws_bits[1]), "the two gate paths give different weight bits"


@pytest.mark.parametrize("E,k", [(16, 4), (128, 4), (200, 8)], ids=["E16", "E128", "E200"])
@pytest.mark.parametrize("path", ["two_phase", "one_phase"])
def test_nan_logits_rank_last(E, k, path, monkeypatch):
    """NaN logits (from NaN or infinite inputs, or a NaN bias) rank after
    every number, NaNs among themselves by id, and get weight 0; the ids
    bit-exact against the oracle on both gate paths, NaN weights where the
    oracle's are NaN, the rest to 1e-5."""
    mm = _mm()
    T, d = 600, 256
    cfg = small_cfg("bf16", T=T, d=d, E=E, k=k, S=0, h=64, tol_y=1e-5)
    inp = make_inputs(cfg, seed=21, gate_only=True)
    rng = np.random.default_rng(22)
    x = inp.x.copy()
    x[rng.choice(T, 20, replace=False), rng.integers(0, d, 20)] = 0x7FC0  # NaN
    x[rng.choice(T, 20, replace=False), rng.integers(0, d, 20)] = 0x7F80  # +inf
    x[rng.choice(T, 20, replace=False), rng.integers(0, d, 20)] = 0xFF80  # -inf
    inp.x = x
    bias = rng.normal(0.0, 0.05, E).astype(np.float32)
    bias[[1, E // 2]] = np.nan
    inp.bias = bias
    monkeypatch.setenv("MOE_GATE_PATH", path)
    say(f"[gate nan] E={E} k={k} path={path}")
    z_ref = oracle.gate_logits(inp.x, inp.wg, inp.bias, nthreads=ORACLE_THREADS)
    idx_ref, w_ref = oracle.select_topk(z_ref, k)
    assert np.isnan(z_ref).any(axis=1).all()  # every token has NaN logits
    shape = mm.shape_of(cfg)
    idx = torch.full((T, k), -3, dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    mm.moe_gate_topk(shape, dev(inp.x), dev(inp.wg), dev(inp.bias), idx, w, None)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), idx_ref)
    got = host(w).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(w_ref))
    fin = ~np.isnan(w_ref)
    assert np.all(got[fin & (w_ref == 0.0)] == 0.0)
    assert rel_l2(got[fin], w_ref[fin]) <= 1e-5


def test_bad_routing_ids_raise_the_device_flag():
    mm = _mm()
    cfg = small_cfg(T=300, d=128, E=8, k=2, S=0, h=64)
    inp = make_inputs(cfg, seed=5, gate_only=True)
    idx = make_routing(cfg.T, cfg.E, cfg.k, seed=6)
    bad = idx.copy()
    bad[3, 1] = cfg.E          # out of range
    bad[10, 0] = -1            # negative
    bad[20, 1] = bad[20, 0]    # repeated expert
    shape = mm.shape_of(cfg)
    T, E, k = cfg.T, cfg.E, cfg.k
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    dest = torch.empty((T, k), dtype=torch.int32, device="cuda")
    src = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    x_perm = torch.zeros((T * k, cfg.d), dtype=torch.bfloat16, device="cuda")
    ws = mm.alloc_workspace(shape, mm.STAGE_DISPATCH)
    mm.moe_dispatch(shape, dev(inp.x), dev(bad), counts, offsets, dest, src, x_perm, None, ws)
    assert mm.moe_get_device_error(ws) == mm.MOE_ERR_BAD_INDEX
    assert mm.moe_get_device_error(ws) == mm.MOE_OK  # reading clears it
    d = host(dest)
    assert d[3, 1] == -1 and d[10, 0] == -1 and d[20, 1] == -1
    valid = np.ones_like(bad, dtype=bool)
    valid[3, 1] = valid[10, 0] = valid[20, 1] = False
    exp_counts = np.bincount(bad[valid], minlength=E)
    assert np.array_equal(host(counts), exp_counts)
    assert host(offsets)[E] == valid.sum()
    # every valid slot got a distinct row inside [0, valid.sum())
    rows = d[valid]
    assert np.array_equal(np.sort(rows), np.arange(valid.sum()))


def test_zero_tokens():
    mm = _mm()
    cfg = small_cfg(T=0, d=128, E=8, k=2, S=1, h=64)
    shape = mm.shape_of(cfg)
    buf = mm.ForwardBuffers(shape)
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((9, 64, 128), dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros((9, 128, 64), dtype=torch.bfloat16, device="cuda")
    wg = torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda")
    buf.run(x, wg, None, w, w, w2)
    torch.cuda.synchronize()


def test_traced_forward_with_some_events_left_out():
    # NULL entries are skipped; the output is the plain forward's
    mm = _mm()
    cfg = small_cfg(T=700, d=256, E=16, k=4, S=1, h=128)
    inp = make_inputs(cfg, seed=9)
    shape = mm.shape_of(cfg)
    args = [dev(inp.x), dev(inp.wg), None, dev(inp.w1), dev(inp.w3), dev(inp.w2)]
    plain = mm.ForwardBuffers(shape)
    plain.run(*args)
    nk = mm.moe_forward_kernel_count(shape)
    names = [mm.moe_forward_kernel_name(shape, i) for i in range(nk)]
    j = names.index("ffn_up")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)]
    for e in ev:
        e.record()  # torch creates the HIP event at its first record
    torch.cuda.synchronize()
    handles = [e.cuda_event if i in (j, j + 1) else None for i, e in enumerate(ev)]
    assert all(h for h in handles if h is not None)
    traced = mm.ForwardBuffers(shape)
    traced.run(*args, events=handles)
    torch.cuda.synchronize()
    assert torch.equal(traced.y, plain.y) and torch.equal(traced.dest_row, plain.dest_row)
    assert ev[j].elapsed_time(ev[j + 1]) > 0.0


@pytest.mark.parametrize("E,k", [(16, 4), (128, 4), (200, 8)], ids=["E16", "E128", "E200"])
@pytest.mark.parametrize("path", ["two_phase", "one_phase"])
def test_tied_logits_go_to_the_lower_id(E, k, path, monkeypatch):
    # gate rows duplicated in pairs: every logit appears twice, and the
    # top-k must list the lower id of a tied pair first (bit-exact vs the
    # oracle, whose tie rule is pinned on the CPU)
    mm = _mm()
    monkeypatch.setenv("MOE_GATE_PATH", path)
    cfg = small_cfg(T=300, d=128, E=E, k=k, S=0, h=64)
    inp = make_inputs(cfg, seed=11)
    inp.wg[1::2] = inp.wg[0::2][: E // 2]
    z = oracle.gate_logits(inp.x, inp.wg, None, nthreads=ORACLE_THREADS)
    oidx, ow = oracle.select_topk(z, k)
    assert np.any(z[:, 0] == z[:, 1])
    idx = torch.empty((cfg.T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, k), dtype=torch.float32, device="cuda")
    mm.moe_gate_topk(mm.shape_of(cfg), dev(inp.x), dev(inp.wg), None, idx, w, None)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), oidx)
    assert rel_l2(host(w), ow) <= 1e-5
