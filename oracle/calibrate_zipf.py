"""Derive the Zipf offset strength of the skewed E=128 top-4 workload.

The workload biases expert e's gate logit by -alpha * s * ln(e + 1) (s = 1.2)
so that the hottest expert takes about 85-90 % of the top-1 picks, the skew of
the trace in the lpnh.cn deep dive (section 2.3: 89 % on one expert after 5k
steps) and the DeepEP notes (section 8.1: hot experts draw 60-80 %). This
script finds alpha by bisection on the oracle's own gate over the first 4096
tokens and prints it; the value is stored as moe_workloads.ZIPF_ALPHA.

Run: python oracle/calibrate_zipf.py
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402
from moe_workloads import CONFIGS, ZIPF_S, make_inputs, zipf_bias  # noqa: E402

N_TOK = 4096
TARGET = 0.875


def top1_share(z, alpha, E):
    zb = (z + zipf_bias(E, alpha, ZIPF_S)[None, :]).astype(np.float32)
    idx, _ = oracle.select_topk(zb, 1)
    return float(np.mean(idx[:, 0] == 0))


def main():
    cfg = CONFIGS["zipf_stress_bf16"]
    inp = make_inputs(cfg, gate_only=True)
    z = oracle.gate_logits(inp.x[:N_TOK], inp.wg, None, nthreads=os.cpu_count())
    lo, hi = 0.0, 10.0
    for _ in range(40):
        mid = (lo + hi) / 2
        if top1_share(z, mid, cfg.E) < TARGET:
            lo = mid
        else:
            hi = mid
    alpha = round(hi, 2)
    print(f"alpha={alpha} top1_share={top1_share(z, alpha, cfg.E):.4f}")


if __name__ == "__main__":
    main()
