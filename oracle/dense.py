"""Whole-batch form of the oracle's expert stage and layer output (test
infrastructure only, like the rest of this package).

The per-token oracle (``layer_tokens`` in moe_oracle.c) applies each expert
FFN to one token row at a time with scalar float64 loops, which is too slow
for every token of the large workloads. This module computes the same
definition for all tokens at once, with one float64 matrix product per
expert over the rows that chose it:

    y[t] = sum_s FFN_{E+s}(x[t]) + sum_j w[t,j] FFN_{e_j}(xq[t]),
    FFN_g(v) = W2_g (silu(W1_g v) * (W3_g v)),  silu(a) = a / (1 + e^-a)

-- the gate-weighted sum of the chosen experts' outputs of
"Deepseek-MoE同步税本质与四层实战优化指南" (gsyq.cn), section 2.3, with the
always-on shared experts of "DeepSeek 中 MoE 的同步税" (wmrh.cn), section 2.1,
and the FFN applied per expert as the DeepEP notes' expert stage
(zzszmyf.github.io, section 7). The matrix product is a library step
(numpy / BLAS in float64); nothing else is blocked or reordered. Gating,
top-k, the fp8 map and the dispatch order are the C oracle's functions.

Pinned against the per-token C oracle (``layer_tokens``, ``expert_rows``),
an independent implementation of the same definition, on small cases of
every workload kind (tests/test_oracle_dense.py).
"""

from __future__ import annotations

import dataclasses

import numpy as np


def _f64(a):
    """float64, float32 or bf16-bit-pattern array -> float64 (exact)."""
    if a.dtype == np.float64:
        return a
    if a.dtype == np.float32:
        return a.astype(np.float64)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class _Threads:
    """Limits BLAS threads to n within the block (n falsy: leave as is)."""

    def __init__(self, n):
        self.n = n
        self.ctx = None

    def __enter__(self):
        if self.n:
            try:
                from threadpoolctl import threadpool_limits
                self.ctx = threadpool_limits(limits=int(self.n))
            except ImportError:  # pragma: no cover
                self.ctx = None
        return self

    def __exit__(self, *exc):
        if self.ctx is not None:
            self.ctx.restore_original_limits()
        return False


def swiglu_rows(v, w1g, w3g, w2g):
    """FFN of one expert group applied to float64 rows v [n, d] -> [n, d]:
    W2 (silu(W1 v) * (W3 v)), every product a float64 matrix product."""
    a = v @ _f64(w1g).T
    b = v @ _f64(w3g).T
    with np.errstate(over="ignore"):
        hmid = a / (1.0 + np.exp(-a)) * b
    return hmid @ _f64(w2g).T


def _dequant(codes, qp):
    from . import fp8_dequantize
    return fp8_dequantize(codes, qp)


def token_inputs(inp, nthreads=None):
    """float64 routed-expert input of every token [T, d]: the row itself, or
    (fp8 dispatch) the row quantised with its own per-token affine map and
    mapped back as code * scale + centre (gsyq.cn section 3.1) -- or, in the
    per-token symmetric absmax mode ("token_absmax"), the same map over the
    symmetric range [-max|x|, max|x|] (centre 0)."""
    from . import fp8_quantize
    if inp.cfg.dispatch != "fp8":
        return _f64(inp.x)
    if getattr(inp.cfg, "quant", "token") == "token_absmax":
        q, qp = fp8_quantize(inp.x, ranges=symmetric_ranges(_as_f32(inp.x)), nthreads=nthreads or 1)
    else:
        q, qp = fp8_quantize(inp.x, nthreads=nthreads or 1)
    return _dequant(q, qp)


def routed_input(inp, tokens, ranges=None, xq=None, nthreads=None):
    """float64 input rows of the routed experts for the given tokens: the
    rows themselves, or (fp8 dispatch) the rows quantised with the per-token
    affine map -- or with the given (min, max) ranges [n, 2] -- and mapped
    back as code * scale + centre (gsyq.cn section 3.1). xq: token_inputs(),
    used when no ranges are given."""
    from . import fp8_quantize
    if ranges is None and xq is not None:
        return xq[tokens]
    x = inp.x[tokens]
    if inp.cfg.dispatch != "fp8":
        return _f64(x)
    q, qp = fp8_quantize(x, ranges=ranges, nthreads=nthreads or 1)
    return _dequant(q, qp)


def routed_rows(inp, offsets, src_token, chunk=4096, nthreads=None, qranges=None, xq=None):
    """The routed experts' output rows in dispatch order, one chunk at a time.

    For expert e the rows offsets[e] .. offsets[e+1]-1 hold the tokens
    src_token[...] (the dispatch order); each chunk is yielded as
    (row0, row1, out [row1-row0, d] float64) with out[r] = FFN_e(xq[token]).
    qranges [rows, 2] (optional, fp8): the (min, max) range each row is
    quantised with (per-expert or global quantiser modes). xq: token_inputs().
    """
    E = len(offsets) - 1
    with _Threads(nthreads):
        for e in range(E):
            lo, hi = int(offsets[e]), int(offsets[e + 1])
            for r0 in range(lo, hi, chunk):
                r1 = min(hi, r0 + chunk)
                toks = np.asarray(src_token[r0:r1], dtype=np.int64)
                rng = None if qranges is None else qranges[r0:r1]
                v = routed_input(inp, toks, rng, xq, nthreads)
                yield r0, r1, swiglu_rows(v, inp.w1[e], inp.w3[e], inp.w2[e])


def shared_rows(inp, tokens, nthreads=None):
    """sum_s FFN_{E+s}(x[t]) for the listed tokens, float64 [n, d]."""
    cfg = inp.cfg
    v = _f64(inp.x[tokens])
    out = np.zeros((len(tokens), cfg.d))
    with _Threads(nthreads):
        for s in range(cfg.S):
            g = cfg.E + s
            out += swiglu_rows(v, inp.w1[g], inp.w3[g], inp.w2[g])
    return out


def layer_dense(inp, nthreads=None, route=None, qrange=None, chunk=4096, gate=None, xq=None,
                tokens=None):
    """Whole-layer output for every token: (topk_idx [T,k], topk_w [T,k]
    float64, y [T,d] float64), the same quantities as layer_tokens over all
    tokens.

    route [T,k] (optional): the expert whose row each slot got under a
    capacity limit, -1 = dropped (contributes nothing; a reassigned slot keeps
    its gate weight). qrange [T,k,2] (optional, fp8): the (min, max) range of
    each slot's row. gate (optional): (topk_idx, topk_w) already computed by
    gate_logits / select_topk for these inputs. xq (optional):
    token_inputs() for these inputs. tokens (optional): compute only these
    tokens' outputs (gate, route, qrange and xq still cover the whole
    batch); the results then have one row per listed token.
    """
    from . import gate_logits, select_topk
    cfg = inp.cfg
    if gate is None:
        z = gate_logits(inp.x, inp.wg, inp.bias, nthreads=nthreads or 1)
        idx, w = select_topk(z, cfg.k)
    else:
        idx, w = gate
    if tokens is not None:
        tokens = np.asarray(tokens, dtype=np.int64)
        sub = dataclasses.replace(inp, cfg=cfg.with_tokens(len(tokens)), x=inp.x[tokens])
        return layer_dense(sub, nthreads, None if route is None else np.asarray(route)[tokens],
                           None if qrange is None else np.asarray(qrange)[tokens], chunk,
                           (idx[tokens], w[tokens]), None if xq is None else xq[tokens])
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    exp_of = idx if route is None else np.asarray(route, dtype=np.int64).reshape(T, k)
    if xq is None and qrange is None:
        xq = token_inputs(inp, nthreads)
    y = np.zeros((T, d))
    with _Threads(nthreads):
        for t0 in range(0, T, chunk):
            t1 = min(T, t0 + chunk)
            y[t0:t1] += shared_rows(inp, np.arange(t0, t1), nthreads=None)
        for e in range(E):
            tt, jj = np.nonzero(exp_of == e)  # token-ascending
            for c0 in range(0, len(tt), chunk):
                t_c, j_c = tt[c0:c0 + chunk], jj[c0:c0 + chunk]
                rng = None if qrange is None else np.asarray(qrange)[t_c, j_c]
                v = routed_input(inp, t_c, rng, xq, nthreads)
                out = swiglu_rows(v, inp.w1[e], inp.w3[e], inp.w2[e])
                contrib = w[t_c, j_c][:, None] * out
                if np.all(np.diff(t_c) > 0):
                    y[t_c] += contrib
                else:  # a reassigned slot may land on an expert its token already has
                    np.add.at(y, t_c, contrib)
    return idx, w, y


def _swiglu_backward_rows(v, g, w1g, w3g, w2g):
    """Backward of one expert group's FFN over float64 rows v [n, d] with
    output gradients g [n, d]: (dv [n, d], dW1 [h, d], dW3 [h, d], dW2 [d, h]).

    Forward: a = W1 v, b = W3 v, u = silu(a) = a sigma(a), hid = u b,
    y = W2 hid. Backward by the chain rule: dhid = W2^T g, da = dhid b silu'(a)
    with silu'(a) = sigma(a) (1 + a (1 - sigma(a))), db = dhid u,
    dv = W1^T da + W3^T db; dW2 = g hid^T, dW1 = da v^T, dW3 = db v^T, summed
    over the rows."""
    W1, W3, W2 = _f64(w1g), _f64(w3g), _f64(w2g)
    a = v @ W1.T
    b = v @ W3.T
    with np.errstate(over="ignore"):
        sg = 1.0 / (1.0 + np.exp(-a))
    u = a * sg
    hid = u * b
    dhid = g @ W2
    da = dhid * b * (sg * (1.0 + a * (1.0 - sg)))
    db = dhid * u
    dv = da @ W1 + db @ W3
    return dv, da.T @ v, db.T @ v, g.T @ hid


def ffn_backward(inp, offsets, src_token, dy_perm, dy_shared=None, xq=None, nthreads=None,
                 chunk=4096):
    """Backward of the grouped expert FFN stage alone, every row at once.

    The routed rows offsets[e] .. offsets[e+1]-1 hold the tokens
    src_token[...] (dispatch order) with input xq[token] (token_inputs: the
    fp8 rows dequantised; the quantiser passes the gradient straight through)
    and output gradient dy_perm[row]; the shared experts see every token's x
    with output gradient dy_shared[t] (the layer output's gradient, weight 1).
    Returns float64 dict(dx_perm [R, d], dx_shared [T, d] or None (the sum
    over the shared experts), dw1 / dw3 [E+S, h, d], dw2 [E+S, d, h]) --
    the gradients returning through the expert stage ("Deepseek-MoE同步税本质与
    四层实战优化指南", gsyq.cn, section 2.4: the backward pass runs the
    exchanges in reverse, the expert computation between them)."""
    cfg = inp.cfg
    E, S, d, h, T = cfg.E, cfg.S, cfg.d, cfg.h, cfg.T
    if xq is None:
        xq = token_inputs(inp, nthreads)
    R = int(offsets[E])
    out = dict(dx_perm=np.zeros((R, d)), dx_shared=np.zeros((T, d)) if S else None,
               dw1=np.zeros((E + S, h, d)), dw3=np.zeros((E + S, h, d)), dw2=np.zeros((E + S, d, h)))
    with _Threads(nthreads):
        for e in range(E):
            for r0 in range(int(offsets[e]), int(offsets[e + 1]), chunk):
                r1 = min(int(offsets[e + 1]), r0 + chunk)
                v = xq[np.asarray(src_token[r0:r1], dtype=np.int64)]
                g = _f64(np.ascontiguousarray(dy_perm[r0:r1]))
                dv, d1, d3, d2 = _swiglu_backward_rows(v, g, inp.w1[e], inp.w3[e], inp.w2[e])
                out["dx_perm"][r0:r1] = dv
                out["dw1"][e] += d1
                out["dw3"][e] += d3
                out["dw2"][e] += d2
        for s in range(S):
            gi = E + s
            for t0 in range(0, T, chunk):
                t1 = min(T, t0 + chunk)
                v = _f64(inp.x[t0:t1])
                g = _f64(np.ascontiguousarray(dy_shared[t0:t1]))
                dv, d1, d3, d2 = _swiglu_backward_rows(v, g, inp.w1[gi], inp.w3[gi], inp.w2[gi])
                out["dx_shared"][t0:t1] += dv
                out["dw1"][gi] += d1
                out["dw3"][gi] += d3
                out["dw2"][gi] += d2
    return out


# ----------------------------------------------------------- fp8 weights ---
# The pages name FP8 for the dispatched activations only ("Deepseek-MoE同步税本质
# 与四层实战优化指南", gsyq.cn, sections 3.1 and 5.2: a per-token min/max map, and
# per-token / per-expert / global modes); weight quantisation is not defined
# there. The reading taken for the fp8-weight variant of the expert stage:
#   * every weight row (one output feature of W1, W3 or W2) gets its own
#     symmetric absmax scale: the same affine map as the activations, applied
#     to the symmetric range [-max|w|, max|w|], so the centre is 0 and the
#     scale is max|w| / 448 (the shared experts' W2 rows jointly over their
#     concatenated blocks);
#   * the shared experts read the same per-token fp8 rows as the routed ones;
#   * the hidden vector silu(a) * b is rounded to bf16 (float32 first) and
#     quantised per row with a symmetric absmax scale over the row's h values
#     (over the S * h values of the shared experts' concatenated blocks) before
#     the down-projection.


def symmetric_ranges(rows):
    """(min, max) = (-max|v|, max|v|) per row of a float array [n, K]."""
    amax = np.max(np.abs(rows), axis=1).astype(np.float32)
    return np.stack([-amax, amax], axis=1)


def _as_f32(a):
    if a.dtype == np.float32:
        return a
    return (a.astype(np.uint32) << 16).view(np.float32)


def quantize_weight_rows(w, nthreads=None):
    """Symmetric absmax e4m3 codes of every row of w [..., K] (bf16 bits or
    float32): (codes uint8 [..., K], scale float32 [...]); the row is
    code * scale."""
    from . import fp8_quantize
    shp = w.shape
    rows = np.ascontiguousarray(w.reshape(-1, shp[-1]))
    q, qp = fp8_quantize(rows, ranges=symmetric_ranges(_as_f32(rows)), nthreads=nthreads or 1)
    assert np.all(qp[:, 1] == 0.0)  # the symmetric range has centre 0
    return q.reshape(shp), qp[:, 0].reshape(shp[:-1])


def quantize_expert_weights(inp, nthreads=None):
    """(q1, s1, q3, s3, q2, s2): every weight row of W1, W3 [G, h, d] and W2
    [G, d, h] as symmetric absmax e4m3 codes with a float32 scale per row.
    The shared experts' W2 rows are quantised jointly: row n of the S
    concatenated blocks [W2_E[n] | ... | W2_{E+S-1}[n]] has one scale (so
    that their down-projections can share one accumulator)."""
    cfg = inp.cfg
    E, S, h = cfg.E, cfg.S, cfg.h
    q1, s1 = quantize_weight_rows(inp.w1, nthreads)
    q3, s3 = quantize_weight_rows(inp.w3, nthreads)
    q2, s2 = quantize_weight_rows(inp.w2, nthreads)
    if S:
        cat = np.concatenate([inp.w2[E + s] for s in range(S)], axis=1)  # [d, S*h]
        qc, sc = quantize_weight_rows(cat, nthreads)
        for s in range(S):
            q2[E + s] = qc[:, s * h:(s + 1) * h]
            s2[E + s] = sc
    return q1, s1, q3, s3, q2, s2


def _deq_rows(q, s):
    from . import fp8_dequantize
    shp = q.shape
    qp = np.zeros((int(np.prod(shp[:-1])), 2), dtype=np.float32)
    qp[:, 0] = s.reshape(-1)
    return fp8_dequantize(q.reshape(-1, shp[-1]), qp).reshape(shp)


def _bf16_round(v64):
    """float64 -> float32 (nearest) -> bf16 (nearest even), as float64."""
    u = v64.astype(np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _quant_hidden(hid, nthreads=None):
    """bf16 hidden rows [n, K] (float64 values) quantised per row with a
    symmetric absmax e4m3 scale, back as float64 code * scale."""
    from . import fp8_dequantize, fp8_quantize
    h32 = hid.astype(np.float32)
    q, qp = fp8_quantize(h32, ranges=symmetric_ranges(h32), nthreads=nthreads or 1)
    return fp8_dequantize(q, qp)


def layer_dense_fp8w(inp, wq, nthreads=None, gate=None, xq=None):
    """Whole-layer output with fp8 expert weights (the reading above):
    (topk_idx, topk_w, y [T, d] float64). wq: quantize_expert_weights(inp).
    Every expert FFN is W2q (Q(bf16(silu(W1q v) * (W3q v)))), Wq the
    dequantised weights and Q the per-row symmetric absmax quantiser, v the
    token's dequantised fp8 row (routed and shared experts alike)."""
    from . import gate_logits, select_topk
    cfg = inp.cfg
    T, d, E, k, S, h = cfg.T, cfg.d, cfg.E, cfg.k, cfg.S, cfg.h
    if gate is None:
        z = gate_logits(inp.x, inp.wg, inp.bias, nthreads=nthreads or 1)
        idx, w = select_topk(z, k)
    else:
        idx, w = gate
    if xq is None:
        xq = token_inputs(inp, nthreads)
    q1, s1, q3, s3, q2, s2 = wq
    y = np.zeros((T, d))

    def up(v, g):
        W1 = _deq_rows(q1[g], s1[g])
        W3 = _deq_rows(q3[g], s3[g])
        a = v @ W1.T
        b = v @ W3.T
        with np.errstate(over="ignore"):
            return _bf16_round(a / (1.0 + np.exp(-a)) * b)

    with _Threads(nthreads):
        if S:
            W2s = [_deq_rows(q2[E + s], s2[E + s]) for s in range(S)]
            for t0 in range(0, T, 4096):
                t1 = min(T, t0 + 4096)
                v = xq[t0:t1]
                hid = np.concatenate([up(v, E + s) for s in range(S)], axis=1)
                hq = _quant_hidden(hid, nthreads)
                for s in range(S):
                    y[t0:t1] += hq[:, s * h:(s + 1) * h] @ W2s[s].T
        for e in range(E):
            tt, jj = np.nonzero(idx == e)
            if len(tt) == 0:
                continue
            W2 = _deq_rows(q2[e], s2[e])
            for c0 in range(0, len(tt), 4096):
                t_c, j_c = tt[c0:c0 + 4096], jj[c0:c0 + 4096]
                hq = _quant_hidden(up(xq[t_c], e), nthreads)
                y[t_c] += w[t_c, j_c][:, None] * (hq @ W2.T)
    return idx, w, y
