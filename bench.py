"""Benchmark: one MoE layer forward (gate -> dispatch -> grouped SwiGLU FFN ->
combine) on one MI355X, through the C ABI.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--detail-configs all|none]
                    [--no-cpu-baseline] [--capacity-factor F [--reassign]]
                    [--quant token|expert|global]
    python bench.py --copy-probe-mib N    # counter calibration, see below

Prints ONE JSON line for the headline workload (default: zipf_stress_bf16,
T=65536, d=4096, E=128 top-4, h=512 -- the largest single-GPU workload by
tokens and bytes). `value` is routed tokens/s, T / (median time of one layer
forward), with every input already resident in HBM.

Timing protocol, per step: write 1 GiB of scratch memory (outside the timed
interval, so the 256 MB Infinity Cache cannot serve the step's inputs from
the previous step), then run one forward whose first and last kernels are
bracketed by HIP events recorded by the library on its stream
(moe_forward_traced). ms_per_step is the median over the K steps, with p10
and p90 beside it. Two more events in the same steps bracket the dominant
kernel, the grouped up-projection, whose mean duration gives the roofline
entry. The other per-kernel durations come from fully traced passes after
the timed region (each recorded event adds a few microseconds to a pass),
also with the flush before each.

--detail-configs all (the default) also times the other large workloads
(deepseekmoe_bf16, coarse_top2_bf16, fp8_dispatch) with the same protocol and
puts their per-stage figures under detail.workloads.

--capacity-factor F caps every routed expert at ceil(F * T*k / E) rows
(overflow dropped, or with --reassign handed to the least-loaded expert);
--quant picks the fp8 rows' range (fp8 workloads only). Both change the
workload, and config names them.

The cpu_baseline leg times the CPU oracle, single-threaded, on a bounded
sample of the same batch (token prefixes until at least 10 s of CPU work).

roofline.traffic is the HBM byte count per launch of the up-projection
measured with the FETCH_SIZE and WRITE_SIZE counters (rocprofv3 --pmc, one
run each), each scaled by what the same counter reads for a plain elementwise
kernel of known size (--copy-probe-mib: reads N MiB, writes N MiB). The
figures live in profiles/traffic_<workload>.txt together with the SHA-256 of
each kernel's source file; a kernel whose source has changed since gets null.
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed tokens/s per MoE layer fwd (1 GPU); dispatch+combine HBM GB/s; FFN MFMA %"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
F32_VEC_PEAK_TFLOPS = 157.3
# the gate's canonical fma chain runs on the non-packed float32 vector units
F32_NONPACKED_PEAK_TFLOPS = 78.6
HEADLINE = "zipf_stress_bf16"
DETAIL_CONFIGS = ["deepseekmoe_bf16", "coarse_top2_bf16", "fp8_dispatch", "fp8_dispatch_fp8w"]
FLUSH_BYTES = 1 << 30

CSRC = "mixture_experts_routing_gemm_amd/csrc/"
# kernel name in the forward -> the source file whose hash a traffic figure is tied to
KERNEL_SOURCES = {
    "gate_topk": CSRC + "gate_common.h",
    "gate_two_phase": CSRC + "gate_two_phase.hip",
    "dispatch_rank": CSRC + "dispatch.hip",
    "dispatch_scan": CSRC + "dispatch.hip",
    "dispatch_permute": CSRC + "dispatch.hip",
    "dispatch_permute_fp8": CSRC + "dispatch.hip",
    "dispatch_map": CSRC + "dispatch.hip",
    "ffn_up": CSRC + "grouped_ffn.hip",
    "ffn_down": CSRC + "grouped_ffn.hip",
    "ffn_hidden_quant": CSRC + "fp8_rows.hip",
    "combine": CSRC + "combine.hip",
}


def algorithmic(cfg, routed=None, gathered=False):
    """Algorithmic bytes / FLOPs of each stage for one layer forward.

    routed: the dispatched rows (T*k unless a capacity limit dropped some).
    The fp8 per-expert and global modes read x once more for the ranges.
    gathered: the forward's up-projection reads its routed rows from x
    through src_token, so its dispatch stage moves only the routing maps;
    "dispatch_rows_bytes" is what the permutation into x_perm moves.
    """
    T, d, E, k, S, h = cfg.T, cfg.d, cfg.E, cfg.k, cfg.S, cfg.h
    R = T * k if routed is None else routed
    b = 4 if cfg.act == "f32" else 2
    bp = 1 if cfg.dispatch == "fp8" else b
    bw = 1 if getattr(cfg, "weights", "act") == "fp8" else b  # bytes per weight
    rows = R + S * T
    xreads = 2 if getattr(cfg, "quant", "token") != "token" else 1
    rows_bytes = (xreads * T * d * b + R * d * bp + 8 * T * k + 4 * T * k
                  + (8 * R if cfg.dispatch == "fp8" else 0))
    return {
        "gate_bytes": T * d * b + E * d * b + 8 * T * k,
        "gate_flops": 2 * T * d * E,
        # ids in, dest_row and src_token out (and, unless gathered, x in and
        # the permuted rows out)
        "dispatch_bytes": 8 * T * k + 4 * R if gathered else rows_bytes,
        "dispatch_rows_bytes": rows_bytes,
        "ffn_up_flops": 4 * rows * d * h,
        # token rows in, both weight matrices of every group, hidden rows out
        "ffn_up_bytes": R * d * bp + S * T * d * (bw if bw == 1 else b) + (E + S) * 2 * h * d * bw
        + rows * h * b + (8 * R if cfg.dispatch == "fp8" else 0),
        "ffn_down_flops": 2 * rows * d * h,
        # hidden rows in, W2 of every group, routed rows and shared sum out
        "ffn_down_bytes": rows * h * (1 if bw == 1 else b) + (E + S) * d * h * bw + R * d * b
        + (T * d * b if S else 0),
        "combine_bytes": R * d * b + (T * d * b if S else 0) + 8 * T * k + T * d * b,
        # backward of combine: dy once, the forward rows in, their gradients out,
        # routing metadata in and the weight gradients out
        "combine_backward_bytes": T * d * b + 2 * R * d * b + 12 * T * k,
        # backward of dispatch: the row gradients and the shared experts' in,
        # the token gradients out
        "dispatch_backward_bytes": R * d * b + (T * d * b if S else 0) + 4 * T * k + T * d * b,
        # backward of the gate: dx read and written, x read once, W_gate read,
        # dW_gate written (float32), w / dw / ids in and the logit gradients out
        # (the per-range partials of dW_gate are not counted)
        "gate_backward_bytes": 3 * T * d * b + E * d * b + 4 * E * d + 16 * T * k,
    }


def _sha(path):
    with open(os.path.join(ROOT, path), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload):
    """{kernel: HBM bytes per launch} from the committed counter summary of
    the workload, for the kernels whose source is unchanged since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return {}
    out = {}
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        parts = line.split()
        # kernel  fetch_kib  write_kib  traffic_bytes  source_sha256
        if len(parts) != 5 or parts[0] == "kernel":
            continue
        name, _, _, traffic, sha = parts
        src = KERNEL_SOURCES.get(name)
        if src is not None and _sha(src) == sha:
            out[name] = int(float(traffic))
    return out


def copy_probe(mib):
    """A plain elementwise kernel that reads and writes `mib` MiB, three times,
    so that the HBM byte counters can be scaled against a known size."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4}))


def host_cpu():
    model = platform.processor() or "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return model, os.cpu_count(), avail


def cpu_baseline(inp, min_s=10.0, max_tokens=None):
    """The oracle's whole layer, one thread, on growing token prefixes of the
    same batch until at least min_s seconds of CPU work."""
    import oracle
    cfg = inp.cfg
    model, ncpu, avail = host_cpu()
    n, dt = 0, 0.0
    step = 16
    cap = cfg.T if max_tokens is None else min(cfg.T, max_tokens)
    t0 = time.perf_counter()
    while dt < min_s and n < cap:
        toks = np.arange(n, min(cap, n + step), dtype=np.int64)
        oracle.layer_tokens(inp, toks, nthreads=1)
        n += len(toks)
        dt = time.perf_counter() - t0
        step = min(step * 2, 256)
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} tokens of the {cfg.name} batch, whole layer per token "
                      f"(float32 gate chain, top-k, float64 SwiGLU experts, weighted sum), "
                      f"1 thread, {dt:.1f} s",
            "host_cpu": model, "host_cpus": ncpu, "cpus_available": avail,
            "cores_used": f"1 of {avail}"}


def backward_leg(mm, torch, cfg, shape, buf, stream, A, x, wg, w1, w3, w2, reps=20):
    """Time the stages of the layer backward on this forward's routing:
    synthetic gradients and expert rows, each launch bracketed by its own
    pair of events (averaged over reps launches); then the expert FFN's
    backward (ffn_backward_leg)."""
    T, d, k = cfg.T, cfg.d, cfg.k
    dt = torch.float32 if cfg.act == "f32" else torch.bfloat16
    g = torch.Generator(device="cuda").manual_seed(7)
    dy = torch.randn((T, d), device="cuda", generator=g).to(dt)
    y_perm = torch.randn((T * k, d), device="cuda", generator=g).to(dt)
    dy_perm = torch.empty((T * k, d), dtype=dt, device="cuda")
    dw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    dx_sh = torch.randn((T, d), device="cuda", generator=g).to(dt) if cfg.S else None
    dx = torch.empty((T, d), dtype=dt, device="cuda")
    dz = torch.empty((T, k), dtype=torch.float32, device="cuda")
    dwg = torch.empty((cfg.E, d), dtype=torch.float32, device="cuda")
    ws_gb = mm.alloc_workspace(shape, mm.STAGE_GATE_BACKWARD)
    calls = {
        "combine_backward": lambda: mm.moe_combine_backward(
            shape, dy, y_perm, buf.dest_row, buf.topk_w, dy_perm, dw, stream),
        "dispatch_backward": lambda: mm.moe_dispatch_backward(
            shape, dy_perm, dx_sh, buf.dest_row, dx, stream),
        "gate_backward": lambda: mm.moe_gate_backward(
            shape, x, wg, buf.topk_idx, buf.topk_w, dw, dz, dx, dwg, ws_gb, stream),
    }
    out = {}
    for name, call in calls.items():
        for _ in range(3):
            call()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        gbps = A[name + "_bytes"] / (ms * 1e-3) / 1e9
        out[name] = {"us": round(ms * 1e3, 2), "GBps": round(gbps, 1),
                     "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "algorithmic_bytes": A[name + "_bytes"]}
    del dy, y_perm, dy_perm, dx_sh, dx, ws_gb
    out["ffn_backward"] = ffn_backward_leg(mm, torch, cfg, shape, buf, stream, x, w1, w3, w2,
                                           reps=max(3, reps // 4))
    return out


def dispatch_leg(mm, torch, cfg, shape, buf, stream, x, flush_cache, nbytes, reps=10):
    """Time moe_dispatch with its permuted rows written out (x_perm), on this
    forward's routing, each call after the cache flush, one event pair
    around each call: the permutation's HBM rate, which the whole-layer
    forward does not pay when its up-projection gathers the rows."""
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    R = T * k
    x_perm = torch.empty((R, d), dtype=torch.bfloat16, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    dest = torch.empty((T, k), dtype=torch.int32, device="cuda")
    src = torch.empty(R, dtype=torch.int32, device="cuda")
    ws_d = mm.alloc_workspace(shape, mm.STAGE_DISPATCH)

    def call():
        mm.moe_dispatch(shape, x, buf.topk_idx, counts, offsets, dest, src, x_perm, None, ws_d,
                        stream)
    call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    torch.cuda.synchronize()
    for i, (a_, b_) in enumerate(ev):
        flush_cache(i)
        a_.record(stream)
        call()
        b_.record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([a_.elapsed_time(b_) for a_, b_ in ev]))
    n = int(offsets[-1].item())
    same = bool(torch.equal(src[:n], buf.src_token[:n]) and torch.equal(dest, buf.dest_row)
                and torch.equal(offsets, buf.offsets))
    del x_perm, counts, offsets, dest, src, ws_d
    torch.cuda.empty_cache()
    return {"us": round(ms * 1e3, 2), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "algorithmic_bytes": nbytes, "maps_equal_forward": same}


def ffn_backward_leg(mm, torch, cfg, shape, buf, stream, x, w1, w3, w2, reps=5):
    """Time moe_grouped_ffn_backward on this forward's dispatch (its rows
    from moe_dispatch, synthetic output gradients): the recomputation of
    a, b and hid, dhid with the SwiGLU backward, dx, and the weight
    gradients. MFMA share counts the 12 * rows * d * h FLOPs of the backward
    proper (the recomputation's 4 * rows * d * h reported beside them)."""
    T, d, E, k, S, h = cfg.T, cfg.d, cfg.E, cfg.k, cfg.S, cfg.h
    fp8 = cfg.dispatch == "fp8"
    R = T * k
    x_perm = torch.empty((R, d), dtype=torch.uint8 if fp8 else torch.bfloat16, device="cuda")
    qp = torch.empty((R, 2), dtype=torch.float32, device="cuda") if fp8 else None
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    dest = torch.empty((T, k), dtype=torch.int32, device="cuda")
    src = torch.empty(R, dtype=torch.int32, device="cuda")
    ws_d = mm.alloc_workspace(shape, mm.STAGE_DISPATCH)
    mm.moe_dispatch(shape, x, buf.topk_idx, counts, offsets, dest, src, x_perm, qp, ws_d, stream)
    rows = int(offsets[-1].item()) + S * T
    g = torch.Generator(device="cuda").manual_seed(9)
    dy_perm = (0.05 * torch.randn((R, d), device="cuda", generator=g)).to(torch.bfloat16)
    dy_sh = (0.05 * torch.randn((T, d), device="cuda", generator=g)).to(torch.bfloat16) if S else None
    dx_perm = torch.empty((R, d), dtype=torch.bfloat16, device="cuda")
    dx_sh = torch.empty((T, d), dtype=torch.bfloat16, device="cuda") if S else None
    G = E + S
    dw1 = torch.empty((G, h, d), dtype=torch.float32, device="cuda")
    dw3 = torch.empty((G, h, d), dtype=torch.float32, device="cuda")
    dw2 = torch.empty((G, d, h), dtype=torch.float32, device="cuda")
    ws = mm.alloc_workspace(shape, mm.STAGE_FFN_BACKWARD)

    def call():
        mm.moe_grouped_ffn_backward(shape, x_perm, qp, offsets, x if S else None, w1, w3, w2,
                                    dy_perm, dy_sh, dx_perm, dx_sh, dw1, dw3, dw2, ws, stream)
    call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    torch.cuda.synchronize()
    for a_, b_ in ev:
        a_.record(stream)
        call()
        b_.record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([a_.elapsed_time(b_) for a_, b_ in ev]))
    flops = 12 * rows * d * h
    peak = BF16_PEAK_TFLOPS
    res = {"us": round(ms * 1e3, 2), "rows": rows, "backward_flops": flops,
           "recompute_flops": 4 * rows * d * h,
           "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
           "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / peak, 4),
           "mfma_frac_incl_recompute": round(16 * rows * d * h / (ms * 1e-3) / 1e12 / peak, 4)}
    if mm.moe_ffn_saved_bytes(shape) > 0:
        # the same backward from activations saved by moe_grouped_ffn_save
        # (no recomputation); the saving forward is not timed here
        saved = mm.alloc_saved(shape)
        y_perm = torch.empty((R, d), dtype=torch.bfloat16, device="cuda")
        y_sh = torch.empty((T, d), dtype=torch.bfloat16, device="cuda") if S else None
        mm.moe_grouped_ffn_save(shape, x_perm, qp, offsets, x if S else None, w1, w3, w2, y_perm, y_sh,
                                saved, mm.alloc_workspace(shape, mm.STAGE_FFN), stream)

        def call_saved():
            mm.moe_grouped_ffn_backward_saved(shape, x_perm, qp, offsets, x if S else None, w1, w3, w2,
                                              saved, dy_perm, dy_sh, dx_perm, dx_sh, dw1, dw3, dw2, ws,
                                              stream)
        call_saved()
        torch.cuda.synchronize()
        for a_, b_ in ev:
            a_.record(stream)
            call_saved()
            b_.record(stream)
        torch.cuda.synchronize()
        ms2 = float(np.median([a_.elapsed_time(b_) for a_, b_ in ev]))
        res["saved_activations"] = {"us": round(ms2 * 1e3, 2),
                                    "tflops": round(flops / (ms2 * 1e-3) / 1e12, 1),
                                    "mfma_frac": round(flops / (ms2 * 1e-3) / 1e12 / peak, 4),
                                    "saved_bytes": mm.moe_ffn_saved_bytes(shape)}
        del saved, y_perm, y_sh
    del x_perm, qp, dy_perm, dy_sh, dx_perm, dx_sh, dw1, dw3, dw2, ws, ws_d
    torch.cuda.empty_cache()
    return res


def _pct(a, q):
    return round(float(np.percentile(a, q)), 5) if len(a) else None


def run_workload(cfg, steps, warmup, flush, with_backward=False, keep_host=False):
    """Times one workload: K flushed steps with events around the forward and
    the up-projection, then fully traced passes for the per-kernel split."""
    import torch

    import mixture_experts_routing_gemm_amd as mm
    from moe_workloads import make_inputs

    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    inp = make_inputs(cfg)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    x, wg, w1, w3, w2 = dev(inp.x), dev(inp.wg), dev(inp.w1), dev(inp.w3), dev(inp.w2)
    bias = None if inp.bias is None else dev(inp.bias)
    if not keep_host:
        inp = None
    shape = mm.shape_of(cfg)
    buf = mm.ForwardBuffers(shape)
    stream = torch.cuda.current_stream()
    fp8w = getattr(cfg, "weights", "act") == "fp8"
    if fp8w:
        # fp8 expert weights: quantised once, before anything is timed
        G = cfg.E + cfg.S
        w1q = torch.empty((G, cfg.h, cfg.d), dtype=torch.uint8, device="cuda")
        w3q = torch.empty_like(w1q)
        w2q = torch.empty((G, cfg.d, cfg.h), dtype=torch.uint8, device="cuda")
        wsc = torch.empty(mm.moe_fp8_weight_scale_floats(shape), dtype=torch.float32, device="cuda")
        mm.moe_quantize_weights(shape, w1, w3, w2, w1q, w3q, w2q, wsc, stream)
        ws8 = mm.alloc_workspace(shape, mm.STAGE_FORWARD_FP8W)
        names = [mm.moe_forward_kernel_name(shape, 0)] + list(mm.FP8W_KERNELS[1:])

        def forward(events=None):
            mm.moe_forward_fp8w(shape, x, wg, bias, w1q, w3q, w2q, wsc, buf.y, buf.topk_idx,
                                buf.topk_w, buf.counts, buf.offsets, buf.dest_row, buf.src_token,
                                ws8, stream, events)
    else:
        names = [mm.moe_forward_kernel_name(shape, i) for i in range(mm.moe_forward_kernel_count(shape))]

        def forward(events=None):
            buf.run(x, wg, bias, w1, w3, w2, events=events)
    nk = len(names)

    def flush_cache(i):
        flush.fill_(i & 0xFF)

    for i in range(warmup):
        flush_cache(i)
        forward()
    torch.cuda.synchronize()

    def make_events(n):
        """n sets of nk+1 events, created (and recorded once) up front"""
        out = []
        for _ in range(n):
            row = [torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)]
            for e in row:
                e.record(stream)
            out.append(row)
        torch.cuda.synchronize()
        return out

    j_up = names.index("ffn_up")
    keep = (0, j_up, j_up + 1, nk)
    evs = make_events(steps)
    handles = [[e.cuda_event if j in keep else None for j, e in enumerate(row)] for row in evs]
    n_tr = min(steps, 10)
    evs_tr = make_events(n_tr)
    handles_tr = [[e.cuda_event for e in row] for row in evs_tr]

    print(f"[bench] {cfg.name}: timing {steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        flush_cache(i)
        forward(handles[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert mm.moe_get_device_error(ws8 if fp8w else buf.ws) == mm.MOE_OK
    step_ms = np.array([row[0].elapsed_time(row[nk]) for row in evs])
    up_ms = np.array([row[j_up].elapsed_time(row[j_up + 1]) for row in evs])

    for i in range(n_tr):
        flush_cache(i)
        forward(handles_tr[i])
    torch.cuda.synchronize()
    per_kernel = np.array([[row[j].elapsed_time(row[j + 1]) for j in range(nk)] for row in evs_tr])
    kmean = dict(zip(names, per_kernel.mean(axis=0).tolist()))

    routed = int(buf.offsets[-1].item())
    gathered = "dispatch_map" in names
    A = algorithmic(cfg, routed, gathered)
    ms_med = float(np.median(step_ms))
    gate_name = names[0]
    t_gate = kmean[gate_name]
    gate_flop_rate = A["gate_flops"] / (t_gate * 1e-3) / 1e12
    t_disp = sum(v for n, v in kmean.items() if n.startswith("dispatch"))
    t_up, t_down = float(np.mean(up_ms)), kmean["ffn_down"]
    t_ffn = t_up + t_down + kmean["ffn_plan"] + kmean.get("ffn_hidden_quant", 0.0)
    t_comb = kmean["combine"]
    gemm_peak = (FP8_PEAK_TFLOPS if fp8w else BF16_PEAK_TFLOPS) if cfg.act == "bf16" else F32_VEC_PEAK_TFLOPS
    res = {
        "T": cfg.T,
        "value": round(cfg.T / (ms_med * 1e-3), 1),
        "ms_per_step": round(ms_med, 5),
        "step_ms_p10_median_p90": [_pct(step_ms, 10), _pct(step_ms, 50), _pct(step_ms, 90)],
        "wall_s_timed_loop_incl_flush": round(wall, 4),
        "kernel_ms": {n: round(v, 5) for n, v in kmean.items()},
        "ffn_up_ms_timed_steps": round(t_up, 5),
        "gate_us": round(t_gate * 1e3, 2),
        "gate_kernel": gate_name,
        "gate_tflops": round(gate_flop_rate, 3),
        "gate_GBps": round(A["gate_bytes"] / (t_gate * 1e-3) / 1e9, 1),
        "dispatch_us": round(t_disp * 1e3, 2),
        "dispatch_GBps": round(A["dispatch_bytes"] / (t_disp * 1e-3) / 1e9, 1),
        "dispatch_hbm_frac": round(A["dispatch_bytes"] / (t_disp * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "ffn_us": round(t_ffn * 1e3, 2),
        "ffn_mfma_frac": round((A["ffn_up_flops"] + A["ffn_down_flops"]) / (t_ffn * 1e-3) / 1e12
                               / gemm_peak, 4),
        "ffn_up_mfma_frac": round(A["ffn_up_flops"] / (t_up * 1e-3) / 1e12 / gemm_peak, 4),
        "ffn_down_mfma_frac": round(A["ffn_down_flops"] / (t_down * 1e-3) / 1e12 / gemm_peak, 4),
        "combine_us": round(t_comb * 1e3, 2),
        "combine_GBps": round(A["combine_bytes"] / (t_comb * 1e-3) / 1e9, 1),
        "combine_hbm_frac": round(A["combine_bytes"] / (t_comb * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "routed_assignments_per_s": round(cfg.T * cfg.k / (ms_med * 1e-3), 1),
        "dispatched_rows": routed,
    }
    if gate_name == "gate_two_phase":
        # the logits' FLOPs run on the bf16 matrix cores (plus the candidates' chains)
        res["gate_frac_of_bf16_peak"] = round(gate_flop_rate / BF16_PEAK_TFLOPS, 4)
    else:
        # every logit is a canonical fma chain on the non-packed float32 vector units
        res["gate_frac_of_f32_nonpacked_peak"] = round(gate_flop_rate / F32_NONPACKED_PEAK_TFLOPS, 4)
    res["gemm_peak_tflops"] = gemm_peak
    if gathered:
        res["rows_gathered_in_ffn_up"] = True
        res["dispatch_materialized"] = dispatch_leg(mm, torch, cfg, shape, buf, stream, x,
                                                    flush_cache, A["dispatch_rows_bytes"])
    extra = {"A": A, "t_up": t_up, "gemm_peak": gemm_peak}
    if with_backward and not fp8w:
        res["backward_stages"] = backward_leg(mm, torch, cfg, shape, buf, stream, A, x, wg,
                                              w1, w3, w2)
    del x, wg, w1, w3, w2, bias, buf
    if fp8w:
        del w1q, w3q, w2q, wsc, ws8
    torch.cuda.empty_cache()
    return res, extra, inp


def detail_config(configs, name):
    """a workload by name; <name>_fp8w is <name> with fp8 expert weights"""
    if name.endswith("_fp8w"):
        return dataclasses.replace(configs[name[:-5]], weights="fp8", name=name)
    return configs[name]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=HEADLINE)
    ap.add_argument("--detail-configs", default="all", choices=["all", "none"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0)
    ap.add_argument("--capacity-factor", type=float, default=0.0)
    ap.add_argument("--reassign", action="store_true")
    ap.add_argument("--quant", default="token", choices=["token", "expert", "global", "token_absmax"])
    ap.add_argument("--fp8-weights", action="store_true",
                    help="fp8 expert weights on the fp8 matrix cores (fp8-row workloads)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the tokens on one GPU; "
              "multi-GPU runs are not implemented", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib)
        return

    import torch

    from moe_workloads import CONFIGS

    cfg = CONFIGS[args.config]
    if args.capacity_factor > 0:
        cap = math.ceil(args.capacity_factor * cfg.T * cfg.k / cfg.E)
        cfg = dataclasses.replace(cfg, capacity=cap, reassign=args.reassign)
    if args.quant != "token":
        if cfg.dispatch != "fp8":
            sys.exit("--quant needs a workload with fp8 dispatch")
        cfg = dataclasses.replace(cfg, quant=args.quant)
    if args.fp8_weights:
        if cfg.dispatch != "fp8":
            sys.exit("--fp8-weights needs a workload with fp8 dispatch")
        cfg = dataclasses.replace(cfg, weights="fp8", name=cfg.name + "_fp8w")
    torch.cuda.set_device(0)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")

    res, ex, inp = run_workload(cfg, args.steps, args.warmup, flush,
                                with_backward=not args.no_backward,
                                keep_host=not args.no_cpu_baseline)
    A = ex["A"]
    up_tflops = A["ffn_up_flops"] / (ex["t_up"] * 1e-3) / 1e12
    plain = not cfg.capacity and cfg.quant == "token" and cfg.weights == "act"
    traffic = measured_traffic(cfg.name) if plain else {}
    detail = dict(res)
    for key in ("value", "ms_per_step", "T"):
        detail.pop(key)
    detail["timing"] = (f"per step: 1 GiB scratch write outside the timed interval, then one "
                        f"forward between HIP events recorded on the library's stream; "
                        f"ms_per_step = median of {args.steps} steps; kernel_ms from "
                        f"{min(args.steps, 10)} fully traced passes (ffn_up: the timed steps)")
    detail["traffic_bytes_per_launch"] = traffic or None
    detail["algorithmic"] = {k: v for k, v in A.items() if not k.endswith("backward_bytes")}
    if args.detail_configs == "all" and args.config == HEADLINE and plain:
        detail["workloads"] = {}
        for name in DETAIL_CONFIGS:
            r, _, _ = run_workload(detail_config(CONFIGS, name), max(5, args.steps // 2),
                                   max(2, args.warmup // 2), flush)
            detail["workloads"][name] = r
    out = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 weights, bf16 activations" if cfg.weights == "fp8" else cfg.act,
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k,
                   "S": cfg.S, "h": cfg.h, "dispatch": cfg.dispatch,
                   **({"capacity": cfg.capacity, "overflow": "reassign" if cfg.reassign else "drop"}
                      if cfg.capacity else {}),
                   **({"quant": cfg.quant} if cfg.quant != "token" else {}),
                   **({"weights": "fp8"} if cfg.weights == "fp8" else {})},
        "roofline": {
            "kernel": "ffn_up",
            "bound": "mfma",
            "achieved": round(up_tflops, 2),
            "peak": ex["gemm_peak"],
            "unit": "TFLOP/s",
            "frac": round(up_tflops / ex["gemm_peak"], 4),
            "traffic": traffic.get("ffn_up"),
            "algorithmic_bytes": A["ffn_up_bytes"],
        },
        "detail": detail,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
