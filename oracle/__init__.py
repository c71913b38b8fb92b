"""CPU oracle for one MoE layer's forward pass (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg import this package. The HIP library never loads it, and it never loads
the HIP library. The per-token arithmetic lives in ``moe_oracle.c`` (plain C,
compiled with gcc -O2 -ffp-contract=off, FMA from the hardware instruction,
no fast-math); its loops over tokens or rows may be split over threads, and
each result is computed the same way whichever thread runs it. ``dense.py``
applies each expert to all of its rows with float64 matrix products (the
whole-batch checks) and holds the fp8-weight variant. This module marshals
numpy arrays into the C code.

Parity status of each function (what pins it, besides itself) is listed in the
``test_oracle_*.py`` tests; every function here has at least one pin.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

F32, BF16 = 0, 1

_c_i64p = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile moe_oracle.c into libmoe_oracle.so next to it."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fno-fast-math",
               "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.oracle_gate_logits.argtypes = [i64, i32, i32, i32, vp, vp, vp, vp, i32]
        L.oracle_select_topk.argtypes = [i64, i32, i32, vp, vp, vp]
        L.oracle_dispatch.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_dispatch_capacity.argtypes = [i64, i32, i32, vp, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_fp8_quantize.argtypes = [i64, i32, i32, vp, vp, vp, i32]
        L.oracle_expert_rows.argtypes = [i32, i32, i32, i64, vp, vp, vp, vp, vp, vp, i32]
        L.oracle_layer_tokens.argtypes = [i32, i32, i32, i32, i32, i32, i32, i64, vp, vp, vp,
                                          vp, vp, vp, vp, vp, vp, vp, vp, vp, i32]
        L.oracle_fp8_quantize_ranges.argtypes = [i64, i32, i32, vp, vp, vp, vp, i32]
        L.oracle_combine_backward.argtypes = [i64, i32, i32, i32, vp, vp, vp, vp, i64, vp, vp]
        L.oracle_dispatch_backward.argtypes = [i64, i32, i32, i32, vp, vp, vp, i64, vp]
        L.oracle_gate_backward.argtypes = [i64, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_layer_backward.argtypes = [i32, i32, i32, i32, i32, i32, i32, i64, vp, vp, vp, vp,
                                            vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_combine.argtypes = [i64, i32, i32, i32, vp, vp, vp, vp, i64, vp]
        L.oracle_bf16_to_float.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_float.restype = ctypes.c_float
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"activation/weight arrays must be float32 or bf16 bits (uint16), got {a.dtype}")


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its input (code {rc})")


def _nthreads(n):
    return int(n) if n else 1


def gate_logits(x, wg, bias=None, nthreads=1):
    """float32 logits [T, E] by one fma chain per (token, expert)."""
    x = np.ascontiguousarray(x)
    wg = np.ascontiguousarray(wg)
    T, d = x.shape
    E = wg.shape[0]
    assert wg.shape[1] == d and wg.dtype == x.dtype
    out = np.empty((T, E), dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    _check(lib().oracle_gate_logits(T, d, E, _dtype_code(x), _p(x), _p(wg), _p(b), _p(out),
                                    _nthreads(nthreads)), "gate_logits")
    return out


def select_topk(logits, k):
    """(topk_idx [T,k] int32, topk_w [T,k] float64) from float32 logits."""
    z = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = z.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    _check(lib().oracle_select_topk(T, E, k, _p(z), _p(idx), _p(w)), "select_topk")
    return idx, w


def gate_topk(x, wg, k, bias=None, nthreads=1):
    z = gate_logits(x, wg, bias, nthreads)
    idx, w = select_topk(z, k)
    return idx, w, z


def dispatch(topk_idx, E, capacity=0, reassign=False, return_route=False):
    """counts [E], offsets [E+1], dest_row [T,k], src_token [T*k] (int32).

    capacity > 0: each expert takes at most that many assignments in token
    order; the overflow is dropped, or with reassign=True handed one at a
    time to the least-loaded expert (ties to the lower id) while any is below
    the cap. Dropped slots get dest_row -1 and no row; src_token holds
    offsets[E] meaningful entries (the rest are -1 here). return_route adds
    route [T,k]: the expert whose row each slot got, -1 if dropped.
    """
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = idx.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    dest = np.empty((T, k), dtype=np.int32)
    src = np.full(T * k, -1, dtype=np.int32)
    route = idx.copy()
    if capacity:
        _check(lib().oracle_dispatch_capacity(T, E, k, _p(idx), int(capacity), int(bool(reassign)),
                                              _p(counts), _p(offsets), _p(dest), _p(src),
                                              _p(route)), "dispatch_capacity")
    else:
        _check(lib().oracle_dispatch(T, E, k, _p(idx), _p(counts), _p(offsets), _p(dest),
                                     _p(src)), "dispatch")
    if return_route:
        return counts, offsets, dest, src, route
    return counts, offsets, dest, src


def e4m3_decode(code: int) -> float:
    return lib().oracle_e4m3_decode(int(code) & 0xFF)


def e4m3_encode(v: float) -> int:
    return int(lib().oracle_e4m3_encode(float(v)))


def fp8_quantize(x, nthreads=1, ranges=None):
    """Per-row affine e4m3 codes [T,d] uint8 and qparams [T,2] float32 (s, c).

    ranges [T,2] (optional): the (min, max) each row is mapped from -- its
    expert's or the batch's in the per-expert and global quantiser modes;
    by default the row's own min/max.
    """
    x = np.ascontiguousarray(x)
    T, d = x.shape
    q = np.empty((T, d), dtype=np.uint8)
    qp = np.empty((T, 2), dtype=np.float32)
    if ranges is not None:
        r = np.ascontiguousarray(ranges, dtype=np.float32).reshape(T, 2)
        _check(lib().oracle_fp8_quantize_ranges(T, d, _dtype_code(x), _p(x), _p(r), _p(q), _p(qp),
                                                _nthreads(nthreads)), "fp8_quantize_ranges")
        return q, qp
    _check(lib().oracle_fp8_quantize(T, d, _dtype_code(x), _p(x), _p(q), _p(qp),
                                     _nthreads(nthreads)), "fp8_quantize")
    return q, qp


def fp8_dequantize(q, qp):
    """float64 dequantised rows q*s + c (the oracle's reading of the map)."""
    table = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[q] * qp[:, 0:1].astype(np.float64) + qp[:, 1:2].astype(np.float64)


def expert_rows(rows, group, w1, w3, w2, nthreads=1):
    """Apply SwiGLU expert group[r] to float64 row r: [n,d] -> [n,d] float64."""
    rows = np.ascontiguousarray(rows, dtype=np.float64)
    group = np.ascontiguousarray(group, dtype=np.int32)
    n, d = rows.shape
    h = w1.shape[1]
    assert w1.shape[2] == d and w2.shape[1:] == (d, h)
    out = np.empty((n, d), dtype=np.float64)
    _check(lib().oracle_expert_rows(d, h, _dtype_code(w1), n, _p(group), _p(rows), _p(w1),
                                    _p(w3), _p(w2), _p(out), _nthreads(nthreads)),
           "expert_rows")
    return out


def layer_tokens(inp, tokens, nthreads=1, route=None, qrange=None):
    """Whole-layer output for the listed tokens: (topk_idx, topk_w, y float64).

    route [n, k] (int, optional): under a capacity limit, the expert whose
    row each slot got (-1: dropped, contributes nothing; a reassigned slot
    keeps its gate weight). It depends on the whole batch's routing, so the
    caller takes it from dispatch(..., capacity, return_route=True).
    qrange [n, k, 2] (optional, fp8 rows): the (min, max) range each slot's
    row is quantised with -- its expert's or the batch's in the per-expert
    and global quantiser modes; by default each token's own.
    """
    cfg = inp.cfg
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    n = tokens.shape[0]
    idx = np.empty((n, cfg.k), dtype=np.int32)
    w = np.empty((n, cfg.k), dtype=np.float64)
    y = np.empty((n, cfg.d), dtype=np.float64)
    b = None if inp.bias is None else np.ascontiguousarray(inp.bias, dtype=np.float32)
    _check(lib().oracle_layer_tokens(cfg.d, cfg.E, cfg.k, cfg.S, cfg.h, _dtype_code(inp.x),
                                     1 if cfg.dispatch == "fp8" else 0, n, _p(tokens),
                                     _p(None if route is None else
                                        np.ascontiguousarray(route, dtype=np.int32).reshape(n, cfg.k)),
                                     _p(None if qrange is None else
                                        np.ascontiguousarray(qrange, dtype=np.float32).reshape(n, cfg.k, 2)),
                                     _p(inp.x),
                                     _p(inp.wg), _p(b), _p(inp.w1), _p(inp.w3), _p(inp.w2),
                                     _p(idx), _p(w), _p(y), _nthreads(nthreads)), "layer_tokens")
    return idx, w, y


def layer_backward(inp, tokens, dy, route=None):
    """Gradients of sum(dy * y) over the listed tokens (small sizes):
    dict of dx [n,d], dtopk_w [n,k] and, summed over the tokens, dwg [E,d],
    dw1 / dw3 [E+S,h,d], dw2 [E+S,d,h] -- all float64. The top-k choice is
    held fixed, fp8 rows pass the gradient straight through, and route
    (optional, -1 = dropped) gives each slot's expert as in layer_tokens."""
    cfg = inp.cfg
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    n, d, E, k, S, h = tokens.shape[0], cfg.d, cfg.E, cfg.k, cfg.S, cfg.h
    dy = np.ascontiguousarray(dy, dtype=np.float64).reshape(n, d)
    out = dict(dx=np.zeros((n, d)), dtopk_w=np.zeros((n, k)), dwg=np.zeros((E, d)),
               dw1=np.zeros((E + S, h, d)), dw3=np.zeros((E + S, h, d)), dw2=np.zeros((E + S, d, h)))
    b = None if inp.bias is None else np.ascontiguousarray(inp.bias, dtype=np.float32)
    r = None if route is None else np.ascontiguousarray(route, dtype=np.int32).reshape(n, k)
    _check(lib().oracle_layer_backward(d, E, k, S, h, _dtype_code(inp.x),
                                       1 if cfg.dispatch == "fp8" else 0, n, _p(tokens), _p(r),
                                       _p(inp.x), _p(inp.wg), _p(b), _p(inp.w1), _p(inp.w3),
                                       _p(inp.w2), _p(dy), _p(out["dx"]), _p(out["dtopk_w"]),
                                       _p(out["dwg"]), _p(out["dw1"]), _p(out["dw3"]),
                                       _p(out["dw2"])), "layer_backward")
    return out


def combine_backward(dy, y_perm, dest_row, topk_w):
    """(dy_perm [rows,d] float64, dtopk_w [T,k] float64): the transpose of
    combine; rows no slot points at stay zero."""
    dy = np.ascontiguousarray(dy)
    y_perm = np.ascontiguousarray(y_perm)
    assert dy.dtype == y_perm.dtype
    dest = np.ascontiguousarray(dest_row, dtype=np.int32)
    T, k = dest.shape
    rows, d = y_perm.shape
    w = np.ascontiguousarray(topk_w, dtype=np.float32)
    dyp = np.zeros((rows, d))
    dw = np.zeros((T, k))
    _check(lib().oracle_combine_backward(T, d, k, _dtype_code(dy), _p(dy), _p(y_perm), _p(dest),
                                         _p(w), rows, _p(dyp), _p(dw)), "combine_backward")
    return dyp, dw


def dispatch_backward(dx_perm, dx_shared, dest_row):
    """dx [T,d] float64 = dx_shared + sum_j dx_perm[dest_row[t,j]]."""
    dx_perm = np.ascontiguousarray(dx_perm)
    dest = np.ascontiguousarray(dest_row, dtype=np.int32)
    T, k = dest.shape
    rows, d = dx_perm.shape
    sh = None if dx_shared is None else np.ascontiguousarray(dx_shared)
    out = np.empty((T, d))
    _check(lib().oracle_dispatch_backward(T, d, k, _dtype_code(dx_perm), _p(dx_perm), _p(sh),
                                          _p(dest), rows, _p(out)), "dispatch_backward")
    return out


def gate_backward(x, wg, topk_idx, topk_w, dtopk_w):
    """(dz [T,k], dx_gate [T,d], dwg [E,d]), all float64: the gate's backward
    with the top-k choice held fixed; dz[t,j] is the gradient of the logit of
    expert topk_idx[t,j] (every other logit's is zero)."""
    x = np.ascontiguousarray(x)
    wg = np.ascontiguousarray(wg)
    assert x.dtype == wg.dtype
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = idx.shape
    E, d = wg.shape
    w = np.ascontiguousarray(topk_w, dtype=np.float64)
    dw = np.ascontiguousarray(dtopk_w, dtype=np.float64)
    dz = np.empty((T, k))
    dxg = np.empty((T, d))
    dwg = np.empty((E, d))
    _check(lib().oracle_gate_backward(T, d, E, k, _dtype_code(x), _p(x), _p(wg), _p(idx), _p(w),
                                      _p(dw), _p(dz), _p(dxg), _p(dwg)), "gate_backward")
    return dz, dxg, dwg


def combine(y_perm, y_shared, dest_row, topk_w):
    """float64 y [T,d] = y_sh + sum_j w_j * y_perm[dest_row[t,j]]."""
    y_perm = np.ascontiguousarray(y_perm)
    dest_row = np.ascontiguousarray(dest_row, dtype=np.int32)
    topk_w = np.ascontiguousarray(topk_w, dtype=np.float32)
    T, k = dest_row.shape
    rows, d = y_perm.shape
    ys = None if y_shared is None else np.ascontiguousarray(y_shared)
    if ys is not None:
        assert ys.dtype == y_perm.dtype and ys.shape == (T, d)
    y = np.empty((T, d), dtype=np.float64)
    _check(lib().oracle_combine(T, d, k, _dtype_code(y_perm), _p(y_perm), _p(ys), _p(dest_row),
                                _p(topk_w), rows, _p(y)), "combine")
    return y


def bf16_to_float(bits: int) -> float:
    return lib().oracle_bf16_to_float(int(bits) & 0xFFFF)


def rows_as_f64(x):
    """Activation rows (float32, or bf16 bits) widened to float64."""
    if x.dtype == np.float32:
        return x.astype(np.float64)
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


from .dense import (ffn_backward, layer_dense, layer_dense_fp8w, quantize_expert_weights,  # noqa: E402,F401
                    quantize_weight_rows, routed_rows, shared_rows, swiglu_rows, symmetric_ranges,
                    token_inputs)
