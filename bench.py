"""Benchmark: one MoE layer forward (gate -> dispatch -> grouped SwiGLU FFN ->
combine) on one MI355X, through the C ABI.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]
                    [--capacity-factor F [--reassign]] [--quant token|expert|global]
    python bench.py --copy-probe-mib N    # counter calibration, see below

--capacity-factor F caps every routed expert at ceil(F * T*k / E) rows
(overflow dropped, or with --reassign handed to the least-loaded expert);
--quant picks the fp8 rows' range (fp8 workloads only). Both change the
workload, and config names them.

Prints ONE JSON line. `value` is routed tokens/s (T / time per layer forward)
with every input already resident in HBM. The library records HIP events on
its stream between kernels (moe_forward_traced): in the timed steps only the
two around the dominant kernel, the grouped up-projection (bf16 matrix cores),
whose mean duration gives the roofline entry; the other per-kernel durations
come from fully traced passes right after the timed region (every recorded
event adds a few microseconds to a pass).
The cpu_baseline leg times the CPU oracle, single-threaded, on a bounded
sample of the same workload.

roofline.traffic is the HBM byte count per launch of that kernel measured
with the FETCH_SIZE and WRITE_SIZE counters (rocprofv3 --pmc, one run each),
each scaled by what the same counter reads for a plain elementwise kernel of
known size (--copy-probe-mib: reads N MiB, writes N MiB). The figures live in
profiles/<kernel>_<workload>_traffic.txt together with the SHA-256 of the
kernel's source file; when the source has changed since, traffic is null.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed tokens/s per MoE layer fwd (1 GPU); dispatch+combine HBM GB/s; FFN MFMA %"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
F32_VEC_PEAK_TFLOPS = 157.3


def algorithmic(cfg, routed=None):
    """Algorithmic bytes / FLOPs of each stage for one layer forward.

    routed: the dispatched rows (T*k unless a capacity limit dropped some).
    The fp8 per-expert and global modes read x once more for the ranges.
    """
    T, d, E, k, S, h = cfg.T, cfg.d, cfg.E, cfg.k, cfg.S, cfg.h
    R = T * k if routed is None else routed
    b = 4 if cfg.act == "f32" else 2
    bp = 1 if cfg.dispatch == "fp8" else b
    rows = R + S * T
    xreads = 2 if getattr(cfg, "quant", "token") != "token" else 1
    return {
        "gate_bytes": T * d * b + E * d * b + 8 * T * k,
        "gate_flops": 2 * T * d * E,
        "dispatch_bytes": xreads * T * d * b + R * d * bp + 8 * T * k + 4 * T * k
        + (8 * R if cfg.dispatch == "fp8" else 0),
        "ffn_up_flops": 4 * rows * d * h,
        # token rows in, both weight matrices of every group, hidden rows out
        "ffn_up_bytes": R * d * bp + S * T * d * b + (E + S) * 2 * h * d * b + rows * h * b
        + (8 * R if cfg.dispatch == "fp8" else 0),
        "ffn_down_flops": 2 * rows * d * h,
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


TRAFFIC_SOURCES = {"ffn_up": "mixture_experts_routing_gemm_amd/csrc/grouped_ffn.hip"}


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None if
    there is none or the kernel's source changed after it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    src = TRAFFIC_SOURCES.get(kernel)
    if src is None or not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    with open(os.path.join(ROOT, src), "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if kv.get("kernel_source_sha256") != sha or "traffic_bytes_per_launch" not in kv:
        return None
    return int(float(kv["traffic_bytes_per_launch"]))


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


def cpu_baseline(cfg, n_tokens):
    import oracle
    from moe_workloads import make_inputs
    inp = make_inputs(cfg)
    toks = np.arange(min(n_tokens, cfg.T), dtype=np.int64)
    t0 = time.perf_counter()
    oracle.layer_tokens(inp, toks, nthreads=1)
    dt = time.perf_counter() - t0
    return {"value": round(len(toks) / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {len(toks)} tokens of the {cfg.name} batch, whole layer per token "
                      f"(float32 gate chain, top-k, float64 SwiGLU experts, weighted sum), "
                      f"1 thread, {dt:.1f} s"}


def backward_leg(mm, torch, cfg, shape, buf, stream, A, x, wg, reps=20):
    """Time the two data-movement stages of the layer backward on this
    forward's routing: synthetic gradients and expert rows, each launch
    bracketed by its own pair of events (averaged over reps launches)."""
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
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="deepseekmoe_bf16")
    ap.add_argument("--cpu-tokens", type=int, default=96)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0)
    ap.add_argument("--capacity-factor", type=float, default=0.0)
    ap.add_argument("--reassign", action="store_true")
    ap.add_argument("--quant", default="token", choices=["token", "expert", "global"])
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the tokens on one GPU; "
              "multi-GPU runs are not implemented", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib)
        return

    import torch

    import mixture_experts_routing_gemm_amd as mm
    from moe_workloads import CONFIGS, make_inputs

    import dataclasses
    import math
    cfg = CONFIGS[args.config]
    if args.capacity_factor > 0:
        cap = math.ceil(args.capacity_factor * cfg.T * cfg.k / cfg.E)
        cfg = dataclasses.replace(cfg, capacity=cap, reassign=args.reassign)
    if args.quant != "token":
        if cfg.dispatch != "fp8":
            sys.exit("--quant needs a workload with fp8 dispatch")
        cfg = dataclasses.replace(cfg, quant=args.quant)
    torch.cuda.set_device(0)
    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    inp = make_inputs(cfg)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    x, wg, w1, w3, w2 = dev(inp.x), dev(inp.wg), dev(inp.w1), dev(inp.w3), dev(inp.w2)
    bias = None if inp.bias is None else dev(inp.bias)
    del inp
    shape = mm.shape_of(cfg)
    buf = mm.ForwardBuffers(shape)
    nk = mm.moe_forward_kernel_count(shape)
    names = [mm.moe_forward_kernel_name(shape, i) for i in range(nk)]
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        buf.run(x, wg, bias, w1, w3, w2)
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

    # Timed steps record only the two events around the up-projection (each
    # recorded event adds a few microseconds to a pass); the per-kernel
    # breakdown comes from fully traced passes after the timed region.
    j_up = names.index("ffn_up")
    evs = make_events(args.steps)
    handles = [[e.cuda_event if j in (j_up, j_up + 1) else None for j, e in enumerate(row)]
               for row in evs]
    n_tr = min(args.steps, 10)
    evs_tr = make_events(n_tr)
    handles_tr = [[e.cuda_event for e in row] for row in evs_tr]

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        buf.run(x, wg, bias, w1, w3, w2, events=handles[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert mm.moe_get_device_error(buf.ws) == mm.MOE_OK
    up_ms_timed = float(np.mean([row[j_up].elapsed_time(row[j_up + 1]) for row in evs]))
    # consecutive up-projection starts are one forward apart: the spread of
    # the timed steps without further events
    steps_ms = np.array([evs[i][j_up].elapsed_time(evs[i + 1][j_up]) for i in range(len(evs) - 1)])

    for i in range(n_tr):
        buf.run(x, wg, bias, w1, w3, w2, events=handles_tr[i])
    torch.cuda.synchronize()
    per_kernel = np.array([[row[j].elapsed_time(row[j + 1]) for j in range(nk)] for row in evs_tr])
    step_ms = np.array([row[0].elapsed_time(row[nk]) for row in evs_tr])
    kmean = dict(zip(names, per_kernel.mean(axis=0).tolist()))
    ms_per_step = wall * 1000.0 / args.steps

    routed = int(buf.offsets[-1].item())
    A = algorithmic(cfg, routed)
    bwd = backward_leg(mm, torch, cfg, shape, buf, stream, A, x, wg)
    t_gate = kmean["gate_topk"]
    t_disp = sum(v for n, v in kmean.items() if n.startswith("dispatch"))
    t_up, t_down = up_ms_timed, kmean["ffn_down"]
    t_ffn = t_up + t_down + kmean["ffn_plan"]
    t_comb = kmean["combine"]
    up_tflops = A["ffn_up_flops"] / (t_up * 1e-3) / 1e12
    gemm_peak = BF16_PEAK_TFLOPS if cfg.act == "bf16" else F32_VEC_PEAK_TFLOPS
    detail = {
        "kernel_ms": {n: round(v, 5) for n, v in kmean.items()},
        "kernel_ms_from": f"{n_tr} fully traced passes after the timed region (ffn_up: timed steps)",
        "ffn_up_ms_timed_steps": round(up_ms_timed, 5),
        "step_ms_events_median": round(float(np.median(step_ms)), 5),
        "timed_step_ms_p10_median_p90": ([round(float(np.percentile(steps_ms, q)), 5) for q in (10, 50, 90)]
                                         if len(steps_ms) else None),
        "gate_us": round(t_gate * 1e3, 2),
        "gate_tflops": round(A["gate_flops"] / (t_gate * 1e-3) / 1e12, 3),
        "dispatch_us": round(t_disp * 1e3, 2),
        "dispatch_GBps": round(A["dispatch_bytes"] / (t_disp * 1e-3) / 1e9, 1),
        "dispatch_hbm_frac": round(A["dispatch_bytes"] / (t_disp * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "ffn_us": round(t_ffn * 1e3, 2),
        "ffn_mfma_frac": round((A["ffn_up_flops"] + A["ffn_down_flops"]) / (t_ffn * 1e-3) / 1e12
                               / gemm_peak, 4),
        "ffn_down_tflops": round(A["ffn_down_flops"] / (t_down * 1e-3) / 1e12, 1),
        "combine_us": round(t_comb * 1e3, 2),
        "combine_GBps": round(A["combine_bytes"] / (t_comb * 1e-3) / 1e9, 1),
        "combine_hbm_frac": round(A["combine_bytes"] / (t_comb * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "routed_assignments_per_s": round(cfg.T * cfg.k / (ms_per_step * 1e-3), 1),
        "dispatched_rows": routed,
        "backward_stages": bwd,
    }
    out = {
        "metric": METRIC,
        "value": round(cfg.T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.act,
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k,
                   "S": cfg.S, "h": cfg.h, "dispatch": cfg.dispatch,
                   **({"capacity": cfg.capacity, "overflow": "reassign" if cfg.reassign else "drop"}
                      if cfg.capacity else {}),
                   **({"quant": cfg.quant} if cfg.quant != "token" else {})},
        "roofline": {
            "kernel": "ffn_up",
            "bound": "mfma",
            "achieved": round(up_tflops, 2),
            "peak": gemm_peak,
            "unit": "TFLOP/s",
            "frac": round(up_tflops / gemm_peak, 4),
            # counters were taken on the plain workload only
            "traffic": (measured_traffic("ffn_up", cfg.name)
                        if not cfg.capacity and cfg.quant == "token" else None),
            "algorithmic_bytes": A["ffn_up_bytes"],
        },
        "detail": detail,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
