"""ctypes binding of the C ABI in include/moe.h (argument marshalling only).

Every function here has the name of the C entry point it calls and takes
torch tensors already resident on the GPU; each step of the layer runs in the
HIP kernels of libmoe_mi355x.so. There is no fallback: if the library is
missing, importing this module raises.

torch is imported first on purpose: the library then binds to the HIP runtime
that torch has already loaded, so tensors and streams are shared.
"""

from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_ERR_BAD_INDEX = -5

MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
STAGE_GATE, STAGE_DISPATCH, STAGE_FFN, STAGE_COMBINE, STAGE_FORWARD = 0, 1, 2, 3, 4
STAGE_GATE_BACKWARD = 5
STAGE_FFN_BACKWARD = 6
STAGE_FORWARD_FP8W = 7
FP8W_KERNELS = ["gate_topk", "dispatch_rank", "dispatch_scan", "dispatch_permute_fp8", "ffn_plan",
                "ffn_up", "ffn_hidden_quant", "ffn_down", "combine"]

_DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3}


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class moe_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("S", ctypes.c_int32), ("h", ctypes.c_int32),
                ("act", ctypes.c_int32), ("dispatch", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("overflow", ctypes.c_int32),
                ("quant", ctypes.c_int32)]

    def __repr__(self):
        return (f"moe_shape(T={self.T}, d={self.d}, E={self.E}, k={self.k}, S={self.S}, "
                f"h={self.h}, act={self.act}, dispatch={self.dispatch}, capacity={self.capacity}, "
                f"overflow={self.overflow}, quant={self.quant})")


MOE_OVERFLOW_DROP, MOE_OVERFLOW_REASSIGN = 0, 1
MOE_QUANT_TOKEN, MOE_QUANT_EXPERT, MOE_QUANT_GLOBAL, MOE_QUANT_TOKEN_ABSMAX = 0, 1, 2, 3
_QUANT = {"token": MOE_QUANT_TOKEN, "expert": MOE_QUANT_EXPERT, "global": MOE_QUANT_GLOBAL,
          "token_absmax": MOE_QUANT_TOKEN_ABSMAX}


def make_shape(T, d, E, k, S, h, act="bf16", dispatch=None, capacity=0,
               reassign=False, quant="token") -> moe_shape:
    a = _DTYPES[act] if isinstance(act, str) else int(act)
    if dispatch is None or dispatch == "act":
        dsp = a
    else:
        dsp = _DTYPES[dispatch] if isinstance(dispatch, str) else int(dispatch)
    q = _QUANT[quant] if isinstance(quant, str) else int(quant)
    return moe_shape(int(T), int(d), int(E), int(k), int(S), int(h), a, dsp, int(capacity),
                     MOE_OVERFLOW_REASSIGN if reassign else MOE_OVERFLOW_DROP, q)


def shape_of(cfg) -> moe_shape:
    """moe_shape from a workload config (fields T, d, E, k, S, h, act, dispatch,
    and capacity / reassign / quant if the config has them)."""
    return make_shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.S, cfg.h, cfg.act,
                      "fp8" if cfg.dispatch == "fp8" else None, getattr(cfg, "capacity", 0),
                      getattr(cfg, "reassign", False), getattr(cfg, "quant", "token"))


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python mixture_experts_routing_gemm_amd/build.py`")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sp = ctypes.POINTER(moe_shape)
    L.moe_workspace_bytes.argtypes = [sp, i32]
    L.moe_workspace_bytes.restype = sz
    L.moe_workspace_init.argtypes = [vp, sz, vp]
    L.moe_workspace_init.restype = i32
    L.moe_status_string.argtypes = [i32]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_gate_topk.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_gate_topk.restype = i32
    L.moe_dispatch.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_dispatch.restype = i32
    L.moe_dispatch_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_dispatch_noalloc.restype = i32
    L.moe_grouped_ffn.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_grouped_ffn.restype = i32
    L.moe_combine.argtypes = [sp, vp, vp, vp, vp, vp, vp]
    L.moe_combine.restype = i32
    L.moe_combine_backward.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_combine_backward.restype = i32
    L.moe_dispatch_backward.argtypes = [sp, vp, vp, vp, vp, vp]
    L.moe_dispatch_backward.restype = i32
    L.moe_gate_backward.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_grouped_ffn_backward.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           vp, vp, sz, vp]
    L.moe_grouped_ffn_backward.restype = i32
    L.moe_ffn_saved_bytes.argtypes = [sp]
    L.moe_ffn_saved_bytes.restype = sz
    L.moe_grouped_ffn_save.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp]
    L.moe_grouped_ffn_save.restype = i32
    L.moe_grouped_ffn_backward_saved.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp,
                                                 vp, vp, vp, vp, sz, vp]
    L.moe_grouped_ffn_backward_saved.restype = i32
    L.moe_gate_backward.restype = i32
    L.moe_forward.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_forward.restype = i32
    L.moe_forward_traced.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     sz, vp, ctypes.POINTER(vp), i32]
    L.moe_forward_traced.restype = i32
    L.moe_fp8_weight_scale_floats.argtypes = [sp]
    L.moe_fp8_weight_scale_floats.restype = sz
    L.moe_quantize_weights.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_quantize_weights.restype = i32
    L.moe_forward_fp8w.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                   sz, vp, ctypes.POINTER(vp), i32]
    L.moe_forward_fp8w.restype = i32
    L.moe_forward_kernel_count.argtypes = [sp]
    L.moe_forward_kernel_count.restype = i32
    L.moe_forward_kernel_name.argtypes = [sp, i32]
    L.moe_forward_kernel_name.restype = ctypes.c_char_p
    L.moe_get_device_error.argtypes = [vp, sz, vp]
    L.moe_get_device_error.restype = i32
    return L


lib = _load()

EXPORTS = ["moe_workspace_bytes", "moe_workspace_init", "moe_status_string", "moe_gate_topk",
           "moe_dispatch", "moe_dispatch_noalloc", "moe_grouped_ffn", "moe_combine", "moe_combine_backward",
           "moe_dispatch_backward", "moe_gate_backward", "moe_grouped_ffn_backward", "moe_forward", "moe_forward_traced",
           "moe_forward_kernel_count", "moe_forward_kernel_name", "moe_get_device_error",
           "moe_fp8_weight_scale_floats", "moe_quantize_weights", "moe_forward_fp8w",
           "moe_ffn_saved_bytes", "moe_grouped_ffn_save", "moe_grouped_ffn_backward_saved"]


def status_string(status: int) -> str:
    return lib.moe_status_string(int(status)).decode()


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    if not t.is_cuda:
        raise ValueError("tensors passed to the MoE library must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _s(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ws(ws):
    if ws is None:
        return None, 0
    return _p(ws), ws.numel() * ws.element_size()


def _check(rc, where):
    if rc != MOE_OK:
        raise MoEError(rc, where)


def moe_workspace_bytes(shape: moe_shape, stage: int) -> int:
    return int(lib.moe_workspace_bytes(ctypes.byref(shape), int(stage)))


def moe_workspace_init(ws, stream=None):
    p, n = _ws(ws)
    _check(lib.moe_workspace_init(p, n, _s(stream)), "moe_workspace_init")


def alloc_workspace(shape: moe_shape, stage: int, device="cuda", stream=None):
    """A zero-headed workspace for `stage` (None when the stage needs none)."""
    n = moe_workspace_bytes(shape, stage)
    if n == 0:
        return None
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    moe_workspace_init(ws, stream)
    return ws


def moe_gate_topk(shape, x, w_gate, bias, topk_idx, topk_w, logits=None, stream=None):
    _check(lib.moe_gate_topk(ctypes.byref(shape), _p(x), _p(w_gate), _p(bias), _p(topk_idx),
                             _p(topk_w), _p(logits), _s(stream)), "moe_gate_topk")


def moe_dispatch(shape, x, topk_idx, counts, offsets, dest_row, src_token, x_perm, qparams, ws,
                 stream=None):
    wp, wn = _ws(ws)
    _check(lib.moe_dispatch(ctypes.byref(shape), _p(x), _p(topk_idx), _p(counts), _p(offsets),
                            _p(dest_row), _p(src_token), _p(x_perm), _p(qparams), wp, wn,
                            _s(stream)), "moe_dispatch")


def moe_dispatch_noalloc(shape, x, topk_idx, counts, offsets, dest_row, src_token, x_perm,
                         qparams, stream=None):
    _check(lib.moe_dispatch_noalloc(ctypes.byref(shape), _p(x), _p(topk_idx), _p(counts),
                                    _p(offsets), _p(dest_row), _p(src_token), _p(x_perm),
                                    _p(qparams), _s(stream)), "moe_dispatch_noalloc")


def moe_grouped_ffn(shape, x_perm, qparams, offsets, x, w1, w3, w2, y_perm, y_shared, ws,
                    stream=None):
    wp, wn = _ws(ws)
    _check(lib.moe_grouped_ffn(ctypes.byref(shape), _p(x_perm), _p(qparams), _p(offsets), _p(x),
                               _p(w1), _p(w3), _p(w2), _p(y_perm), _p(y_shared), wp, wn,
                               _s(stream)), "moe_grouped_ffn")


def moe_combine(shape, y_perm, y_shared, dest_row, topk_w, y, stream=None):
    _check(lib.moe_combine(ctypes.byref(shape), _p(y_perm), _p(y_shared), _p(dest_row),
                           _p(topk_w), _p(y), _s(stream)), "moe_combine")


def moe_combine_backward(shape, dy, y_perm, dest_row, topk_w, dy_perm, dtopk_w, stream=None):
    _check(lib.moe_combine_backward(ctypes.byref(shape), _p(dy), _p(y_perm), _p(dest_row),
                                    _p(topk_w), _p(dy_perm), _p(dtopk_w), _s(stream)),
           "moe_combine_backward")


def moe_gate_backward(shape, x, w_gate, topk_idx, topk_w, dtopk_w, dlogits_topk, dx, dw_gate, ws,
                      stream=None):
    wp, wn = _ws(ws)
    _check(lib.moe_gate_backward(ctypes.byref(shape), _p(x), _p(w_gate), _p(topk_idx), _p(topk_w),
                                 _p(dtopk_w), _p(dlogits_topk), _p(dx), _p(dw_gate), wp, wn,
                                 _s(stream)),
           "moe_gate_backward")


def moe_grouped_ffn_backward(shape, x_perm, qparams, offsets, x, w1, w3, w2, dy_perm, dy_shared,
                             dx_perm, dx_shared, dw1, dw3, dw2, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib.moe_grouped_ffn_backward(ctypes.byref(shape), _p(x_perm), _p(qparams), _p(offsets),
                                        _p(x), _p(w1), _p(w3), _p(w2), _p(dy_perm), _p(dy_shared),
                                        _p(dx_perm), _p(dx_shared), _p(dw1), _p(dw3), _p(dw2), wp,
                                        wn, _s(stream)), "moe_grouped_ffn_backward")


def moe_ffn_saved_bytes(shape):
    return int(lib.moe_ffn_saved_bytes(ctypes.byref(shape)))


def alloc_saved(shape, device="cuda"):
    """The caller buffer of activations saved for the backward (uint8)."""
    n = moe_ffn_saved_bytes(shape)
    if n == 0:
        raise MoEError(-2, "moe_ffn_saved_bytes: shape not supported")
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_grouped_ffn_save(shape, x_perm, qparams, offsets, x, w1, w3, w2, y_perm, y_shared, saved,
                         ws, stream=None):
    wp, wn = _ws(ws)
    sp_, sn = _ws(saved)
    _check(lib.moe_grouped_ffn_save(ctypes.byref(shape), _p(x_perm), _p(qparams), _p(offsets), _p(x),
                                    _p(w1), _p(w3), _p(w2), _p(y_perm), _p(y_shared), sp_, sn, wp, wn,
                                    _s(stream)), "moe_grouped_ffn_save")


def moe_grouped_ffn_backward_saved(shape, x_perm, qparams, offsets, x, w1, w3, w2, saved, dy_perm,
                                   dy_shared, dx_perm, dx_shared, dw1, dw3, dw2, ws, stream=None):
    wp, wn = _ws(ws)
    sp_, sn = _ws(saved)
    _check(lib.moe_grouped_ffn_backward_saved(ctypes.byref(shape), _p(x_perm), _p(qparams), _p(offsets),
                                              _p(x), _p(w1), _p(w3), _p(w2), sp_, sn, _p(dy_perm),
                                              _p(dy_shared), _p(dx_perm), _p(dx_shared), _p(dw1),
                                              _p(dw3), _p(dw2), wp, wn, _s(stream)),
           "moe_grouped_ffn_backward_saved")


def moe_dispatch_backward(shape, dx_perm, dx_shared, dest_row, dx, stream=None):
    _check(lib.moe_dispatch_backward(ctypes.byref(shape), _p(dx_perm), _p(dx_shared),
                                     _p(dest_row), _p(dx), _s(stream)), "moe_dispatch_backward")


def moe_forward(shape, x, w_gate, bias, w1, w3, w2, y, topk_idx, topk_w, counts, offsets,
                dest_row, src_token, ws, stream=None):
    wp, wn = _ws(ws)
    _check(lib.moe_forward(ctypes.byref(shape), _p(x), _p(w_gate), _p(bias), _p(w1), _p(w3),
                           _p(w2), _p(y), _p(topk_idx), _p(topk_w), _p(counts), _p(offsets),
                           _p(dest_row), _p(src_token), wp, wn, _s(stream)), "moe_forward")


def moe_forward_traced(shape, x, w_gate, bias, w1, w3, w2, y, topk_idx, topk_w, counts, offsets,
                       dest_row, src_token, ws, events, stream=None):
    """events: a sequence of raw hipEvent_t handles (ints), or None where no
    event is to be recorded."""
    wp, wn = _ws(ws)
    arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(None if e is None else int(e))
                                            for e in events])
    _check(lib.moe_forward_traced(ctypes.byref(shape), _p(x), _p(w_gate), _p(bias), _p(w1),
                                  _p(w3), _p(w2), _p(y), _p(topk_idx), _p(topk_w), _p(counts),
                                  _p(offsets), _p(dest_row), _p(src_token), wp, wn, _s(stream),
                                  arr, len(events)), "moe_forward_traced")


def moe_fp8_weight_scale_floats(shape) -> int:
    return int(lib.moe_fp8_weight_scale_floats(ctypes.byref(shape)))


def moe_quantize_weights(shape, w1, w3, w2, w1q, w3q, w2q, wscale, stream=None):
    _check(lib.moe_quantize_weights(ctypes.byref(shape), _p(w1), _p(w3), _p(w2), _p(w1q), _p(w3q),
                                    _p(w2q), _p(wscale), _s(stream)), "moe_quantize_weights")


def moe_forward_fp8w(shape, x, w_gate, bias, w1q, w3q, w2q, wscale, y, topk_idx, topk_w, counts,
                     offsets, dest_row, src_token, ws, stream=None, events=None):
    wp, wn = _ws(ws)
    if events is None:
        ev, n = None, 0
    else:
        ev = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(None if e is None else int(e))
                                               for e in events])
        n = len(events)
    _check(lib.moe_forward_fp8w(ctypes.byref(shape), _p(x), _p(w_gate), _p(bias), _p(w1q), _p(w3q),
                                _p(w2q), _p(wscale), _p(y), _p(topk_idx), _p(topk_w), _p(counts),
                                _p(offsets), _p(dest_row), _p(src_token), wp, wn, _s(stream), ev, n),
           "moe_forward_fp8w")


def moe_forward_kernel_count(shape) -> int:
    return int(lib.moe_forward_kernel_count(ctypes.byref(shape)))


def moe_forward_kernel_name(shape, i) -> str | None:
    r = lib.moe_forward_kernel_name(ctypes.byref(shape), int(i))
    return None if r is None else r.decode()


def moe_get_device_error(ws, stream=None) -> int:
    """Reads and clears the sticky device flag (synchronises the stream)."""
    wp, wn = _ws(ws)
    return int(lib.moe_get_device_error(wp, wn, _s(stream)))
