"""GPU-vs-oracle parity of the two data-movement stages of the layer backward.

The gradients return along the routing path (gsyq.cn, section 2.4; the
DeepEP notes, section 7, dispatch and combine): the backward of combine sends
w_j * dy[t] to each of token t's expert rows and takes the gate-weight
gradient <dy[t], y_perm[row]>; the backward of dispatch sums each token's
k row gradients (plus the shared experts') back into token order.

Every call goes through the C ABI. Bars, element by element, derived from the
arithmetic (u = 2^-24, the float32 unit roundoff; b = 2^-8, the bf16 one):
  * dy_perm = round(w * dy): one float32 product, then one rounding to the
    activation dtype: |err| <= (2u + b)|ref| for bf16, u|ref| for float32;
  * dtopk_w: a float32 dot product of length d; a lane sums at most
    n = ceil(d / (64 N)) N products in order (N = 8 bf16 or 4 float32 values
    per 16-byte chunk), then a 6-level butterfly adds the lanes' sums:
    |err| <= (n + 8) u sum_c |dy_c y_c|;
  * dx: k + 1 float32 terms summed in slot order and rounded once:
    |err| <= b|ref| + (k + 3) u sum |terms| for bf16 (b -> 0 for float32);
  * rows of dy_perm that no slot maps to are never written (bit-exact).
Inputs come from the seeded generators and the oracle's dispatch, never from
the GPU path.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from gpu_util import act_torch, as_f64, dev, host, requires_gpu, say
from moe_workloads import CONFIGS, make_routing, make_rows, make_weights

pytestmark = [pytest.mark.gpu, requires_gpu]

U = 2.0 ** -24
SENTINEL = 0x7F7F  # bf16 / half of a float32 bit pattern never produced by a product here


def _mm():
    import mixture_experts_routing_gemm_amd as mm
    return mm


# (name, T, d, E, k, act, skew, capacity, reassign)
CASES = [
    ("f32_small", 777, 256, 8, 4, "f32", 0.0, 0, False),
    ("bf16_ragged", 1001, 512, 16, 2, "bf16", 0.0, 0, False),
    ("bf16_k8_wide", 513, 2056, 64, 8, "bf16", 0.0, 0, False),
    ("bf16_drop", 2048, 1024, 32, 4, "bf16", 1.2, 200, False),
    ("bf16_reassign", 2048, 1024, 32, 4, "bf16", 1.2, 260, True),
    ("f32_drop_k1", 999, 64, 4, 1, "f32", 1.5, 100, False),
    ("bf16_one_token", 1, 128, 8, 3, "bf16", 0.0, 0, False),
]


def _routing(T, E, k, skew, capacity, reassign, seed):
    idx = make_routing(T, E, k, seed=seed, skew=skew)
    _, offsets, dest, _ = oracle.dispatch(idx, E, capacity=capacity, reassign=reassign)
    return dest, int(offsets[E])


def _compact(dest, toks):
    """Restrict to the sampled tokens: their slots' rows, renumbered 0.. in
    slot order (dropped slots stay -1); returns (dest_s, source rows)."""
    sub = dest[toks]
    flat = sub.reshape(-1)
    valid = flat >= 0
    dest_s = np.full(flat.shape, -1, dtype=np.int32)
    dest_s[valid] = np.arange(int(valid.sum()), dtype=np.int32)
    return dest_s.reshape(sub.shape), flat[valid].astype(np.int64)


def check_combine_backward(name, T, d, E, k, act, skew, capacity, reassign, toks=None, seed=5):
    mm = _mm()
    dest, nrows = _routing(T, E, k, skew, capacity, reassign, seed)
    rows = T * k
    dy = make_rows(T, d, act, seed=seed + 1)
    y_perm = make_rows(rows, d, act, seed=seed + 2)
    w = make_weights(T, k, seed=seed + 3)
    shape = mm.make_shape(T, d, E, k, 0, 64, act, capacity=capacity, reassign=reassign)

    dt = act_torch(act)
    dyp = torch.empty((rows, d), dtype=dt, device="cuda")
    if act == "bf16":
        dyp.view(torch.int16).fill_(SENTINEL)
    else:
        dyp.view(torch.int32).fill_(SENTINEL << 16 | SENTINEL)
    dw = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    say(f"[backward {name}] combine_backward T={T} d={d} E={E} k={k} {act} rows={nrows}")
    mm.moe_combine_backward(shape, dev(dy), dev(y_perm), dev(dest), dev(w), dyp, dw)
    torch.cuda.synchronize()
    got_p, got_w = host(dyp), host(dw)

    # rows no slot maps to keep the sentinel
    mapped = np.zeros(rows, dtype=bool)
    mapped[dest[dest >= 0]] = True
    untouched = got_p[~mapped]
    if untouched.size:
        pat = untouched.view(np.uint16) if act == "f32" else untouched
        assert np.all(pat == SENTINEL), "combine_backward wrote a row no slot maps to"

    toks = np.arange(T) if toks is None else toks
    dest_s, src_rows = _compact(dest, toks)
    y_s = y_perm[src_rows]
    ref_p, ref_w = oracle.combine_backward(dy[toks], y_s, dest_s, w[toks])

    got_rows = as_f64(got_p[src_rows])
    b = 2.0 ** -8 if act == "bf16" else 0.0
    err = np.abs(got_rows - ref_p)
    ok = err <= ((2 * U if b else U) + b) * np.abs(ref_p)
    say(f"[backward {name}] dy_perm max rel {np.max(err / np.maximum(np.abs(ref_p), 1e-30)):.3e}")
    assert ok.all(), f"dy_perm: {int((~ok).sum())} elements beyond one rounding"

    # dtopk_w: slot by slot against the float64 dot product
    gw = got_w[toks]
    flat_dest = dest_s.reshape(-1)
    scale = np.zeros(flat_dest.shape)
    dyt = as_f64(dy[toks])
    tok_of_slot = np.repeat(np.arange(len(toks)), k)
    v = flat_dest >= 0
    scale[v] = np.sum(np.abs(dyt[tok_of_slot[v]] * as_f64(y_s[flat_dest[v]])), axis=1)
    per_chunk = 8 if act == "bf16" else 4
    n_lane = -(-d // (64 * per_chunk)) * per_chunk
    bound = (n_lane + 8) * U * scale.reshape(gw.shape)
    werr = np.abs(gw - ref_w)
    say(f"[backward {name}] dtopk_w max err/bound {np.max(werr / np.maximum(bound, 1e-300)):.3f}")
    assert np.all(werr <= bound), "dtopk_w beyond the float32 dot-product bound"
    assert np.all(gw[dest_s < 0] == 0.0), "a dropped slot's weight gradient is not zero"


def check_dispatch_backward(name, T, d, E, k, act, skew, capacity, reassign, shared=True,
                            toks=None, seed=9):
    mm = _mm()
    dest, nrows = _routing(T, E, k, skew, capacity, reassign, seed)
    rows = max(nrows, 1)
    dxp = make_rows(rows, d, act, seed=seed + 1)
    dxs = make_rows(T, d, act, seed=seed + 2) if shared else None
    shape = mm.make_shape(T, d, E, k, 0, 64, act, capacity=capacity, reassign=reassign)
    dx = torch.empty((T, d), dtype=act_torch(act), device="cuda")
    say(f"[backward {name}] dispatch_backward T={T} d={d} E={E} k={k} {act} shared={shared}")
    mm.moe_dispatch_backward(shape, dev(dxp), None if dxs is None else dev(dxs), dev(dest), dx)
    torch.cuda.synchronize()
    got = as_f64(host(dx))

    toks = np.arange(T) if toks is None else toks
    dest_s, src_rows = _compact(dest, toks)
    sh = None if dxs is None else dxs[toks]
    ref = oracle.dispatch_backward(dxp[src_rows], sh, dest_s)
    # sum of |terms| per element
    absum = np.zeros_like(ref) if sh is None else np.abs(as_f64(sh))
    rows64 = np.abs(as_f64(dxp[src_rows]))
    for j in range(k):
        r = dest_s[:, j]
        m = r >= 0
        absum[m] += rows64[r[m]]
    b = 2.0 ** -8 if act == "bf16" else 0.0
    bound = b * np.abs(ref) + (k + 3) * U * absum
    err = np.abs(got[toks] - ref)
    say(f"[backward {name}] dx max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3f}")
    assert np.all(err <= bound), "dx beyond one rounding of the float32 sum"


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_combine_backward(case):
    check_combine_backward(*case)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("shared", [True, False])
def test_dispatch_backward(case, shared):
    check_dispatch_backward(*case, shared=shared)


def test_backward_empty_batch():
    """T = 0 is a no-op that touches nothing (NULL pointers are allowed)."""
    mm = _mm()
    shape = mm.make_shape(0, 128, 8, 2, 0, 64, "bf16")
    mm.moe_combine_backward(shape, None, None, None, None, None, None)
    mm.moe_dispatch_backward(shape, None, None, None, None)


def test_backward_null_pointer_rejected():
    mm = _mm()
    shape = mm.make_shape(4, 128, 8, 2, 0, 64, "bf16")
    t = torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mm.MoEError):
        mm.moe_combine_backward(shape, t, None, None, None, t, None)
    with pytest.raises(mm.MoEError):
        mm.moe_dispatch_backward(shape, None, None, None, t)


@pytest.mark.parametrize("name", ["deepseekmoe_bf16", "coarse_top2_bf16"])
def test_backward_full_size(name):
    """At a workload's full size and routing shape (uniform routing of its
    T, d, E, k), checked on sampled tokens."""
    cfg = CONFIGS[name]
    rng = np.random.default_rng(4)
    toks = np.unique(np.concatenate([[0, 1, cfg.T // 2, cfg.T - 1],
                                     rng.integers(0, cfg.T, 1500)])).astype(np.int64)
    args = (name, cfg.T, cfg.d, cfg.E, cfg.k, cfg.act, 0.0, cfg.capacity, cfg.reassign)
    check_combine_backward(*args, toks=toks)
    check_dispatch_backward(*args, shared=True, toks=toks)


# ---------------------------------------------------------------------------
# Backward of the gate (top-k choice held fixed). Bars, element by element:
#  * dz = w (dw - sum_l w_l dw_l): a float32 butterfly sum of k products and
#    two more roundings: |err| <= bz = 10 u w (|dw| + sum_l |w_l dw_l|);
#  * dx = act(dx0 + sum_j dz_j Wg[e_j]): b|ref| + (k + 3) u sum|terms|, plus
#    sum_j bz_j |Wg[e_j]| for the error dz carries in;
#  * dWg[e] = sum of dz x over e's slots in float32 (token order within a
#    range of tokens, then the ranges' partials in order):
#    (N_e + 2) u sum|dz x| + sum bz |x|, N_e = slots on expert e; two calls
#    give the same bits;
#  * every element of dWg is written (a NaN fill must not survive).

# (name, T, d, E, k, act)
GATE_CASES = [
    ("bf16_small", 1000, 512, 16, 4, "bf16"),
    ("f32_small", 333, 256, 8, 2, "f32"),
    ("bf16_ragged_cols", 517, 2056, 64, 8, "bf16"),
    ("bf16_E256", 300, 384, 256, 8, "bf16"),
    ("bf16_E128", 600, 320, 128, 4, "bf16"),
    ("f32_E100", 300, 96, 100, 3, "f32"),
    ("bf16_top1", 200, 128, 8, 1, "bf16"),
    ("bf16_one_token", 1, 64, 4, 2, "bf16"),
    # the matrix-core weight gradient (bf16, d % 256 == 0): plane rows of
    # 768 features (E = 256), padded planes (E = 100), ragged chunks
    ("bf16_mfma_E256", 700, 512, 256, 8, "bf16"),
    ("bf16_mfma_E100", 1500, 768, 100, 3, "bf16"),
]


def _scatter(idx, vals, E):
    T, k = idx.shape
    D = np.zeros((T, E))
    for j in range(k):
        D[np.arange(T), idx[:, j]] += vals[:, j]
    return D


def check_gate_backward(name, T, d, E, k, act, with_dx=True, seed=21, skew=0.0, repeat=False):
    mm = _mm()
    x = make_rows(T, d, act, seed=seed)
    wg = make_rows(E, d, act, seed=seed + 1)
    idx = make_routing(T, E, k, seed=seed + 2, skew=skew)
    if repeat:
        # one expert in two slots of every third token: both slots' terms count
        idx[::3, 1] = idx[::3, 0]
    w = make_weights(T, k, seed=seed + 3)
    rng = np.random.default_rng(seed + 4)
    dw = rng.standard_normal((T, k)).astype(np.float32)
    dw[rng.random((T, k)) < 0.05] = 0.0  # some slots dropped
    dx0 = make_rows(T, d, act, seed=seed + 5)
    shape = mm.make_shape(T, d, E, k, 0, 64, act)
    dz = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    dx = dev(dx0) if with_dx else None
    dwg = torch.full((E, d), float("nan"), dtype=torch.float32, device="cuda")
    say(f"[gate-backward {name}] T={T} d={d} E={E} k={k} {act} dx={with_dx}")
    ws = mm.alloc_workspace(shape, mm.STAGE_GATE_BACKWARD)
    mm.moe_gate_backward(shape, dev(x), dev(wg), dev(idx), dev(w), dev(dw), dz, dx, dwg, ws)
    torch.cuda.synchronize()

    z_ref, dxg_ref, dwg_ref = oracle.gate_backward(x, wg, idx, w.astype(np.float64),
                                                   dw.astype(np.float64))
    w64, dw64 = w.astype(np.float64), dw.astype(np.float64)
    bz = 10 * U * w64 * (np.abs(dw64) + np.sum(np.abs(w64 * dw64), axis=1, keepdims=True))
    gz = host(dz).astype(np.float64)
    assert np.all(np.abs(gz - z_ref) <= bz), "dz beyond its float32 bound"

    xa, wga = np.abs(as_f64(x)), np.abs(as_f64(wg))
    if with_dx:
        ref = as_f64(dx0) + dxg_ref
        terms = np.abs(as_f64(dx0)) + _scatter(idx, np.abs(z_ref), E) @ wga
        b = 2.0 ** -8 if act == "bf16" else 0.0
        bound = b * np.abs(ref) + (k + 3) * U * terms + _scatter(idx, bz, E) @ wga
        err = np.abs(as_f64(host(dx)) - ref)
        say(f"[gate-backward {name}] dx max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3f}")
        assert np.all(err <= bound), "dx beyond its bound"

    got_wg = host(dwg).astype(np.float64)
    again = torch.full_like(dwg, float("nan"))
    mm.moe_gate_backward(shape, dev(x), dev(wg), dev(idx), dev(w), dev(dw), dz, None, again, ws)
    torch.cuda.synchronize()
    assert torch.equal(again, dwg), "dw_gate differs between two calls"
    assert np.all(np.isfinite(got_wg)), "dw_gate has unwritten elements"
    n_e = np.bincount(idx.reshape(-1), minlength=E).astype(np.float64)[:, None]
    bound = (n_e + 2) * U * (_scatter(idx, np.abs(z_ref), E).T @ xa) + _scatter(idx, bz, E).T @ xa
    err = np.abs(got_wg - dwg_ref)
    say(f"[gate-backward {name}] dw_gate max err/bound {np.max(err / np.maximum(bound, 1e-300)):.3f}")
    assert np.all(err <= bound), "dw_gate beyond its float32 bound"


@pytest.mark.parametrize("case", GATE_CASES, ids=[c[0] for c in GATE_CASES])
def test_gate_backward(case):
    check_gate_backward(*case)


def test_gate_backward_without_dx():
    check_gate_backward("no_dx", 700, 256, 32, 6, "bf16", with_dx=False)


@pytest.mark.parametrize("d", [256, 200], ids=["mfma", "lds"])
def test_gate_backward_repeated_expert(d):
    # both weight-gradient paths sum every slot of an expert, also when a
    # token lists it twice
    check_gate_backward(f"repeat_d{d}", 900, d, 16, 4, "bf16", repeat=True)


def test_gate_backward_empty_batch_clears_dw_gate():
    mm = _mm()
    shape = mm.make_shape(0, 256, 8, 2, 0, 64, "bf16")
    dwg = torch.full((8, 256), float("nan"), dtype=torch.float32, device="cuda")
    ws = mm.alloc_workspace(shape, mm.STAGE_GATE_BACKWARD)
    mm.moe_gate_backward(shape, None, None, None, None, None, None, None, dwg, ws)
    torch.cuda.synchronize()
    assert torch.all(dwg == 0).item()


@pytest.mark.parametrize("name", ["deepseekmoe_bf16", "coarse_top2_bf16", "zipf_stress_bf16",
                                  "fp8_dispatch"])
def test_gate_backward_full_size(name):
    # zipf_stress_bf16 with routing as skewed as its gate's (expert 0 in
    # about 85 % of the tokens' top-1; most experts nearly empty);
    # fp8_dispatch's gate backward is bf16 (k = 6)
    cfg = CONFIGS[name]
    skew = 3.0 if name == "zipf_stress_bf16" else 0.0
    check_gate_backward(name, cfg.T, cfg.d, cfg.E, cfg.k, cfg.act, skew=skew)
