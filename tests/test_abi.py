"""The C-ABI library loads, exports every declared symbol, and validates its
arguments on the host (no GPU is touched by anything in this file)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "mixture_experts_routing_gemm_amd", "libmoe_mi355x.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def mm():
    import mixture_experts_routing_gemm_amd as m
    return m


def test_library_exports_every_declared_symbol(mm):
    names = declared_functions()
    assert len(names) >= 12
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(mm.EXPORTS)


def test_status_strings(mm):
    for st in (0, -1, -2, -3, -4, -5):
        assert mm.status_string(st) and mm.status_string(st) != "unknown status"
    assert mm.status_string(7) == "unknown status"


def test_workspace_sizes(mm):
    s = mm.make_shape(4096, 2048, 32, 8, 2, 1408, "bf16")
    fwd = mm.moe_workspace_bytes(s, mm.STAGE_FORWARD)
    # y_perm + H (routed and shared) + y_sh at least: with bf16 rows on the
    # 256 x 256 tiles the up-projection gathers its rows from x, so the whole
    # layer's forward holds no x_perm
    need = 4096 * 8 * 2048 * 2 + 4096 * (8 + 2) * 1408 * 2 + 4096 * 2048 * 2
    assert need < fwd < need + (1 << 20)
    # fp8 rows are written out by dispatch: x_perm (1 byte a value) and its
    # (scale, centre) pairs as well
    s8 = mm.make_shape(4096, 2048, 32, 8, 2, 1408, "bf16", dispatch="fp8")
    need8 = need + 4096 * 8 * 2048 + 4096 * 8 * 8
    assert need8 < mm.moe_workspace_bytes(s8, mm.STAGE_FORWARD) < need8 + (1 << 20)
    # shapes off the 256 x 256 tiles (h % 128 != 0) keep x_perm
    so = mm.make_shape(4096, 2048, 32, 8, 2, 1400, "bf16")
    needo = 4096 * 8 * 2048 * 2 * 2 + 4096 * (8 + 2) * 1400 * 2 + 4096 * 2048 * 2
    assert needo < mm.moe_workspace_bytes(so, mm.STAGE_FORWARD) < needo + (1 << 20)
    assert mm.moe_workspace_bytes(s, mm.STAGE_GATE) == 0
    assert mm.moe_workspace_bytes(s, mm.STAGE_COMBINE) == 0
    # one float32 [E, d] partial per token range, at least one range
    gb = mm.moe_workspace_bytes(s, mm.STAGE_GATE_BACKWARD)
    assert gb >= 256 + s.E * s.d * 4 and gb % 256 == 0
    assert 0 < mm.moe_workspace_bytes(s, mm.STAGE_DISPATCH) < (1 << 20)
    bad = mm.make_shape(4096, 2048, 300, 8, 2, 1408, "bf16")
    assert mm.moe_workspace_bytes(bad, mm.STAGE_FORWARD) == 0
    assert mm.moe_workspace_bytes(s, 99) == 0


def _raw(mm):
    return mm._binding.lib


FAKE = 0x100000  # an aligned, never-dereferenced address: every call below fails validation


@pytest.mark.parametrize("kw,status", [
    (dict(E=300), -2), (dict(k=9, E=16), -2), (dict(k=5, E=4), -1), (dict(T=-1), -1),
    (dict(S=9), -2), (dict(d=100), -2), (dict(d=200, dispatch=2), -2), (dict(act=2), -2),
    (dict(dispatch=2, act=0), -2), (dict(d=0), -1), (dict(capacity=-1), -1),
    (dict(capacity=4, overflow=2), -1), (dict(quant=1), -1), (dict(quant=4, dispatch=2), -1),
])
def test_forward_rejects_bad_shapes(mm, kw, status):
    base = dict(T=64, d=256, E=8, k=2, S=1, h=128, act=1, dispatch=None, capacity=0, overflow=0,
                quant=0)
    base.update(kw)
    s = mm.make_shape(base["T"], base["d"], base["E"], base["k"], base["S"], base["h"],
                      base["act"], base["dispatch"], base["capacity"])
    s.overflow = base["overflow"]
    s.quant = base["quant"]
    p = ctypes.c_void_p(FAKE)
    rc = _raw(mm).moe_forward(ctypes.byref(s), p, p, None, p, p, p, p, p, p, p, p, p, p, p,
                              1 << 40, None)
    assert rc == status


def test_null_misaligned_and_workspace_errors(mm):
    lib = _raw(mm)
    s = mm.make_shape(64, 256, 8, 2, 0, 128, "bf16")
    p = ctypes.c_void_p(FAKE)
    odd = ctypes.c_void_p(FAKE + 8)
    assert lib.moe_gate_topk(ctypes.byref(s), None, p, None, p, p, None, None) == -1
    assert lib.moe_gate_topk(ctypes.byref(s), odd, p, None, p, p, None, None) == -1
    assert lib.moe_gate_topk(None, p, p, None, p, p, None, None) == -1
    # dispatch: workspace too small / missing / misaligned
    assert lib.moe_dispatch(ctypes.byref(s), p, p, p, p, p, p, p, None, p, 16, None) == -3
    assert lib.moe_dispatch(ctypes.byref(s), p, p, p, p, p, p, p, None, None, 1 << 30, None) == -3
    assert lib.moe_dispatch(ctypes.byref(s), p, p, p, p, p, p, p, None,
                            ctypes.c_void_p(FAKE + 16), 1 << 30, None) == -3
    # fp8 dispatch needs qparams
    s8 = mm.make_shape(64, 256, 8, 2, 0, 128, "bf16", "fp8")
    assert lib.moe_dispatch(ctypes.byref(s8), p, p, p, p, p, p, p, None, p, 1 << 30, None) == -1
    # shared experts need x and y_shared; no shared experts forbids y_shared
    s1 = mm.make_shape(64, 256, 8, 2, 1, 128, "bf16")
    assert lib.moe_grouped_ffn(ctypes.byref(s1), p, None, p, None, p, p, p, p, p, p, 1 << 30, None) == -1
    assert lib.moe_grouped_ffn(ctypes.byref(s), p, None, p, None, p, p, p, p, p, p, 1 << 30, None) == -1
    assert lib.moe_combine(ctypes.byref(s), p, None, None, p, p, None) == -1
    assert lib.moe_workspace_init(None, 1024, None) == -3
    assert lib.moe_get_device_error(None, 1024, None) == -3


def test_zero_tokens_is_a_no_op(mm):
    # T = 0 validates and returns OK without enqueuing anything
    lib = _raw(mm)
    s = mm.make_shape(0, 256, 8, 2, 1, 128, "bf16")
    p = ctypes.c_void_p(FAKE)
    assert lib.moe_gate_topk(ctypes.byref(s), p, p, None, p, p, None, None) == 0
    assert lib.moe_combine(ctypes.byref(s), p, p, p, p, p, None) == 0
    n = mm.moe_workspace_bytes(s, mm.STAGE_FORWARD)
    assert lib.moe_forward(ctypes.byref(s), p, p, None, p, p, p, p, p, p, p, p, p, p, p, n, None) == 0


def test_traced_forward_needs_enough_events(mm):
    lib = _raw(mm)
    s = mm.make_shape(64, 256, 8, 2, 1, 128, "bf16")
    p = ctypes.c_void_p(FAKE)
    n = mm.moe_forward_kernel_count(s)
    ev = (ctypes.c_void_p * n)(*([FAKE] * n))
    rc = lib.moe_forward_traced(ctypes.byref(s), p, p, None, p, p, p, p, p, p, p, p, p, p, p,
                                1 << 40, None, ev, n)
    assert rc == -1
    assert mm.moe_forward_kernel_name(mm.make_shape(64, 256, 8, 2, 0, 128, "bf16", "fp8"), 3) == \
        "dispatch_permute_fp8"
    assert mm.moe_forward_kernel_name(s, n) is None


def test_backward_entry_points_validate_on_the_host(mm):
    """The three backward stages reject NULL / misaligned pointers and a
    missing or short workspace before anything is enqueued; T = 0 is a no-op
    for the combine and dispatch transposes."""
    lib = _raw(mm)
    s = mm.make_shape(64, 256, 8, 2, 0, 128, "bf16")
    p = ctypes.c_void_p(FAKE)
    odd = ctypes.c_void_p(FAKE + 4)
    sp = ctypes.byref(s)
    # combine backward: every pointer is required
    assert lib.moe_combine_backward(sp, p, p, p, p, p, None, None) == -1
    assert lib.moe_combine_backward(sp, odd, p, p, p, p, p, None) == -1
    assert lib.moe_combine_backward(None, p, p, p, p, p, p, None) == -1
    # dispatch backward: dx_shared is optional, the rest required
    assert lib.moe_dispatch_backward(sp, p, None, None, p, None) == -1
    assert lib.moe_dispatch_backward(sp, p, odd, p, p, None) == -1
    # gate backward: dw_gate and a workspace are always needed
    n = mm.moe_workspace_bytes(s, mm.STAGE_GATE_BACKWARD)
    assert n > 0
    assert lib.moe_gate_backward(sp, p, p, p, p, p, p, None, None, p, n, None) == -1
    assert lib.moe_gate_backward(sp, p, p, p, p, p, p, None, p, None, n, None) == -3
    assert lib.moe_gate_backward(sp, p, p, p, p, p, p, None, p, p, n - 256, None) == -3
    assert lib.moe_gate_backward(sp, p, p, p, p, p, None, None, p, p, n, None) == -1
    assert lib.moe_gate_backward(sp, p, p, p, p, p, p, odd, p, p, n, None) == -1
    # an unsupported shape is refused the same way as by the forward stages
    bad = mm.make_shape(64, 256, 300, 2, 0, 128, "bf16")
    assert lib.moe_combine_backward(ctypes.byref(bad), p, p, p, p, p, p, None) == -2
    z = mm.make_shape(0, 256, 8, 2, 0, 128, "bf16")
    assert lib.moe_combine_backward(ctypes.byref(z), None, None, None, None, None, None, None) == 0
    assert lib.moe_dispatch_backward(ctypes.byref(z), None, None, None, None, None) == 0


def test_saved_activation_entry_points_validate_on_the_host(mm):
    """moe_ffn_saved_bytes: a, b and hid of the routed rows and of the shared
    experts' token rows, each section 256-byte aligned, or 0 off the
    persistent tiles; the save / saved-backward calls refuse such shapes
    and a missing, misaligned or short buffer before anything is enqueued."""
    lib = _raw(mm)
    s = mm.make_shape(64, 256, 8, 2, 1, 128, "bf16")
    # routed: 128 rows x 128 values x 2 bytes, three times; shared: 64 rows
    assert mm.moe_ffn_saved_bytes(s) == 3 * 128 * 128 * 2 + 3 * 64 * 128 * 2
    assert mm.moe_ffn_saved_bytes(mm.make_shape(64, 256, 8, 2, 0, 136, "bf16")) == 0  # h % 128
    assert mm.moe_ffn_saved_bytes(mm.make_shape(64, 64, 8, 2, 0, 128, "f32")) == 0
    n = mm.moe_ffn_saved_bytes(s)
    p = ctypes.c_void_p(FAKE)
    sp = ctypes.byref(s)
    wsn = mm.moe_workspace_bytes(s, mm.STAGE_FFN)
    # save: saved missing, misaligned (16 but not 256 bytes) or short
    assert lib.moe_grouped_ffn_save(sp, p, None, p, p, p, p, p, p, p, None, n, p, wsn, None) == -1
    assert lib.moe_grouped_ffn_save(sp, p, None, p, p, p, p, p, p, p, ctypes.c_void_p(FAKE + 16), n, p,
                                    wsn, None) == -1
    assert lib.moe_grouped_ffn_save(sp, p, None, p, p, p, p, p, p, p, p, n - 256, p, wsn, None) == -1
    bad = mm.make_shape(64, 256, 8, 2, 1, 136, "bf16")
    assert lib.moe_grouped_ffn_save(ctypes.byref(bad), p, None, p, p, p, p, p, p, p, p, n, p, wsn,
                                    None) == -2
    # saved backward: the same checks on `saved`, then the backward's own
    bn = mm.moe_workspace_bytes(s, mm.STAGE_FFN_BACKWARD)
    args = [p, None, p, p, p, p, p]
    tail = [p, p, p, p, p, p, p, p, bn, None]
    assert lib.moe_grouped_ffn_backward_saved(sp, *args, None, n, *tail) == -1
    assert lib.moe_grouped_ffn_backward_saved(sp, *args, p, n - 256, *tail) == -1
    assert lib.moe_grouped_ffn_backward_saved(ctypes.byref(bad), *args, p, n, *tail) == -2
    assert lib.moe_grouped_ffn_backward_saved(sp, *args, p, n, p, p, p, p, p, p, p, p, bn - 256,
                                              None) == -3
