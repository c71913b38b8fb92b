"""moe_dispatch_noalloc (dispatch with its working arrays in a device array
the library owns, for callers that cannot allocate) against moe_dispatch
with a caller workspace, through the C ABI: two calls in a row, the second
with a smaller input, each output bit-identical; and the host-side refusal
of a shape whose working arrays exceed that array."""

from __future__ import annotations

import ctypes
import dataclasses

import numpy as np
import pytest
import torch

from gpu_util import dev, host, requires_gpu, say
from moe_workloads import CONFIGS, make_inputs, make_routing

pytestmark = [pytest.mark.gpu, requires_gpu]


def _mm():
    import mixture_experts_routing_gemm_amd as mm
    return mm


def _outputs(cfg, fp8):
    T, E, k, d = cfg.T, cfg.E, cfg.k, cfg.d
    o = dict(counts=torch.full((E,), -9, dtype=torch.int32, device="cuda"),
             offsets=torch.full((E + 1,), -9, dtype=torch.int32, device="cuda"),
             dest=torch.full((T, k), -9, dtype=torch.int32, device="cuda"),
             src=torch.full((T * k,), -9, dtype=torch.int32, device="cuda"))
    if fp8:
        o["x_perm"] = torch.zeros((T * k, d), dtype=torch.uint8, device="cuda")
        o["qp"] = torch.zeros((T * k, 2), dtype=torch.float32, device="cuda")
    else:
        o["x_perm"] = torch.zeros((T * k, d), dtype=torch.bfloat16, device="cuda")
        o["qp"] = None
    return o


def _same(a, b, n):
    assert torch.equal(a["counts"], b["counts"])
    assert torch.equal(a["offsets"], b["offsets"])
    assert torch.equal(a["dest"], b["dest"])
    assert torch.equal(a["src"][:n], b["src"][:n])
    assert torch.equal(a["x_perm"][:n].view(torch.uint8), b["x_perm"][:n].view(torch.uint8))
    if a["qp"] is not None:
        assert torch.equal(a["qp"][:n].view(torch.int32), b["qp"][:n].view(torch.int32))


CASES = [
    # (workload, T, overrides): the second of each pair is smaller
    ("fp8_dispatch", 6000, dict(d=512, E=64, k=6, S=0, quant="expert", capacity=600, reassign=True)),
    ("fp8_dispatch", 900, dict(d=256, E=16, k=4, S=0)),
    ("zipf_stress_bf16", 20000, dict(d=256, E=128, k=4, capacity=700)),
    ("zipf_stress_bf16", 1234, dict(d=128, E=8, k=2)),
]


@pytest.mark.parametrize("pair", [0, 1])
def test_noalloc_dispatch_matches_workspace_dispatch(pair):
    mm = _mm()
    for name, T, kw in CASES[2 * pair: 2 * pair + 2]:
        cfg = dataclasses.replace(CONFIGS[name], T=T, **kw)
        fp8 = cfg.dispatch == "fp8"
        say(f"[noalloc] {name} T={T} {kw}")
        inp = make_inputs(cfg, seed=9, gate_only=True)
        idx = dev(make_routing(cfg.T, cfg.E, cfg.k, seed=T, skew=1.2))
        x = dev(inp.x)
        shape = mm.shape_of(cfg)
        ref = _outputs(cfg, fp8)
        ws = mm.alloc_workspace(shape, mm.STAGE_DISPATCH)
        mm.moe_dispatch(shape, x, idx, ref["counts"], ref["offsets"], ref["dest"], ref["src"],
                        ref["x_perm"], ref["qp"], ws)
        got = _outputs(cfg, fp8)
        mm.moe_dispatch_noalloc(shape, x, idx, got["counts"], got["offsets"], got["dest"],
                                got["src"], got["x_perm"], got["qp"])
        torch.cuda.synchronize()
        n = int(host(ref["offsets"])[-1])
        assert n > 0
        _same(ref, got, n)
        assert mm.moe_get_device_error(ws) == mm.MOE_OK


def test_noalloc_dispatch_refuses_a_shape_beyond_its_array():
    mm = _mm()
    lib = mm._binding.lib
    s = mm.make_shape(1 << 21, 256, 256, 8, 0, 128, "bf16")
    assert mm.moe_workspace_bytes(s, mm.STAGE_DISPATCH) > (16 << 20)
    p = ctypes.c_void_p(0x100000)  # never dereferenced: refused on the host
    assert lib.moe_dispatch_noalloc(ctypes.byref(s), p, p, p, p, p, p, p, None, None) == \
        mm.MOE_ERR_UNSUPPORTED
    # T = 0 needs no buffers and enqueues nothing
    z = mm.make_shape(0, 256, 8, 2, 0, 128, "bf16")
    assert lib.moe_dispatch_noalloc(ctypes.byref(z), None, None, None, None, None, None, None,
                                    None, None) == mm.MOE_OK
