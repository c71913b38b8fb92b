"""Seeded synthetic workloads for one MoE layer's forward pass.

This module is shared by the tests, the benchmark and the smoke check. It only
draws random numbers and rounds them to the storage dtype; it holds none of the
layer's arithmetic (no gating, routing, FFN or combine), so both the CPU oracle
and the HIP path can take their inputs from here without sharing any logic.

Shapes follow the pages' workloads:
  * tiny fp32 layer (top-2 of 8) -- a correctness case for the routing code in
    "DeepSeek 中 MoE 的同步税" (wmrh.cn), section 4.1;
  * DeepSeekMoE fine-grained layer, 32 routed experts top-8 plus 2 shared
    experts -- same page, section 2.1 (m=4, N=8 expert segmentation; K_s=2);
  * coarse top-2 of 16 at batch 32 x seq 512 x hidden 5120 --
    "Deepseek-MoE同步税本质与四层实战优化指南" (gsyq.cn), section 2.1;
  * E=128 top-4 with a heavily skewed router -- "DeepSeek MoE ... 路由" deep
    dive (lpnh.cn), section 2.2 (E=128, k=4 top-k table) and section 2.3
    (a skewed trace with 89 % of top-1 picks on one expert);
  * FP8 dispatch at hidden 4096 with 64 routed experts top-6 plus 2 shared --
    gsyq.cn section 3.1 (per-token min/max affine FP8) and the DeepEP notes
    (zzszmyf.github.io), section 1 (FP8 tokens at hidden 4096).

Random draws: numpy.random.default_rng(seed) (PCG64), standard normals drawn
in float32, in the fixed order x -> (fp8 config) outlier mask -> gate weight ->
for each expert group g in routed 0..E-1 then shared E..E+S-1: W1_g, W3_g,
W2_g. bf16 storage is the round-to-nearest-even of those float32 draws, done
by torch's CPU cast; bf16 arrays are returned as uint16 bit patterns.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

# Zipf offset strength for the skewed E=128 config. Derived once by
# oracle/calibrate_zipf.py (bisection on the oracle's gate over the first 4096
# tokens of that config) so that expert 0 takes 85-90 % of the top-1 picks.
ZIPF_ALPHA = 2.68
ZIPF_S = 1.2


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    d: int
    E: int
    k: int
    S: int
    h: int
    act: str            # "f32" or "bf16": dtype of x, gate and expert weights, y
    dispatch: str       # "act" (rows keep the activation dtype) or "fp8"
    sigma_x: float = 1.0
    sigma_gate: float = 0.02
    sigma_w: float = 0.02
    zipf_bias: bool = False
    outlier_p: float = 0.0
    outlier_scale: float = 1.0
    # rows each routed expert may hold (0: no limit); beyond it, assignments
    # in token order are dropped, or with reassign handed to the least-loaded
    # expert
    capacity: int = 0
    reassign: bool = False
    # fp8 rows: the rows whose min/max range a row is mapped from ("token",
    # "expert", "global"), or "token_absmax" (each row's symmetric range)
    quant: str = "token"
    # expert weights: "act" (the activation dtype) or "fp8" (e4m3 codes with
    # a scale per row, on the fp8 matrix cores; fp8 rows only)
    weights: str = "act"
    # relative-L2 bound on the layer output y
    tol_y: float = 2e-2

    def with_tokens(self, T: int) -> "MoEConfig":
        return dataclasses.replace(self, T=int(T))

    @property
    def groups(self) -> int:
        return self.E + self.S


CONFIGS = {
    "tiny_fp32": MoEConfig(
        "tiny_fp32", T=256, d=64, E=8, k=2, S=0, h=128, act="f32", dispatch="act",
        sigma_w=1.0 / math.sqrt(64), tol_y=1e-5),
    "deepseekmoe_bf16": MoEConfig(
        "deepseekmoe_bf16", T=4096, d=2048, E=32, k=8, S=2, h=1408, act="bf16",
        dispatch="act", tol_y=2e-2),
    "coarse_top2_bf16": MoEConfig(
        "coarse_top2_bf16", T=16384, d=5120, E=16, k=2, S=0, h=1536, act="bf16",
        dispatch="act", tol_y=2e-2),
    "zipf_stress_bf16": MoEConfig(
        "zipf_stress_bf16", T=65536, d=4096, E=128, k=4, S=0, h=512, act="bf16",
        dispatch="act", zipf_bias=True, tol_y=2e-2),
    "fp8_dispatch": MoEConfig(
        "fp8_dispatch", T=32768, d=4096, E=64, k=6, S=2, h=1024, act="bf16",
        dispatch="fp8", outlier_p=1e-3, outlier_scale=50.0, tol_y=6e-2),
}

# A capacity-limited variant of the skewed workload: capacity factor 1.25,
# i.e. each expert holds at most 1.25 * T*k/E rows (the DeepEP notes, DeepSeek-V3
# load balancing part A, put the factor near 1.0); under the skew most of the
# hottest experts' assignments are dropped. Not one of the five configs: it is
# a parity case for the capacity limit.
CONFIGS["zipf_capacity_bf16"] = MoEConfig(
    "zipf_capacity_bf16", T=16384, d=2048, E=128, k=4, S=0, h=512, act="bf16",
    dispatch="act", zipf_bias=True, capacity=640, tol_y=2e-2)

# The same with the overflow reassigned to the least-loaded expert (the
# option those notes say V3 mainly uses); capacity factor 1.0, so that every
# expert ends with exactly T*k/E rows.
CONFIGS["zipf_reassign_bf16"] = MoEConfig(
    "zipf_reassign_bf16", T=16384, d=2048, E=128, k=4, S=0, h=512, act="bf16",
    dispatch="act", zipf_bias=True, capacity=512, reassign=True, tol_y=2e-2)

# the order the five configs are listed in the workload table
CONFIG_ORDER = ["tiny_fp32", "deepseekmoe_bf16", "coarse_top2_bf16",
                "zipf_stress_bf16", "fp8_dispatch"]


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), round to nearest even."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(a: np.ndarray, act: str) -> np.ndarray:
    if act == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    return to_bf16_bits(a)


def zipf_bias(E: int, alpha: float = ZIPF_ALPHA, s: float = ZIPF_S) -> np.ndarray:
    """Per-expert logit offset -alpha * s * ln(e + 1): expert 0 is the hottest."""
    e = np.arange(E, dtype=np.float64)
    return (-alpha * s * np.log(e + 1.0)).astype(np.float32)


@dataclasses.dataclass
class MoEInputs:
    cfg: MoEConfig
    x: np.ndarray        # [T, d] float32 or bf16 bits
    wg: np.ndarray       # [E, d]
    bias: np.ndarray | None  # [E] float32 or None
    w1: np.ndarray       # [E+S, h, d]
    w3: np.ndarray       # [E+S, h, d]
    w2: np.ndarray       # [E+S, d, h]


def make_inputs(cfg: MoEConfig, seed: int = 0, T: int | None = None,
                gate_only: bool = False) -> MoEInputs:
    """Draw one layer's inputs. T overrides the token count (a different T
    gives a different x draw). gate_only skips the expert weights (x, the
    outlier mask and the gate weight come first in the draw order, so they are
    the same either way)."""
    if T is not None:
        cfg = cfg.with_tokens(T)
    rng = np.random.default_rng(seed)
    G, d, h = cfg.groups, cfg.d, cfg.h
    x = rng.standard_normal((cfg.T, d), dtype=np.float32) * np.float32(cfg.sigma_x)
    if cfg.outlier_p > 0:
        mask = rng.random((cfg.T, d), dtype=np.float32) < cfg.outlier_p
        x = np.where(mask, x * np.float32(cfg.outlier_scale), x).astype(np.float32)
    wg = rng.standard_normal((cfg.E, d), dtype=np.float32) * np.float32(cfg.sigma_gate)
    bias = zipf_bias(cfg.E) if cfg.zipf_bias else None
    if gate_only:
        return MoEInputs(cfg, _store(x, cfg.act), _store(wg, cfg.act), bias, None, None, None)
    wdt = np.float32 if cfg.act == "f32" else np.uint16
    w1 = np.empty((G, h, d), dtype=wdt)
    w3 = np.empty((G, h, d), dtype=wdt)
    w2 = np.empty((G, d, h), dtype=wdt)
    sw = np.float32(cfg.sigma_w)
    for g in range(G):
        w1[g] = _store(rng.standard_normal((h, d), dtype=np.float32) * sw, cfg.act)
        w3[g] = _store(rng.standard_normal((h, d), dtype=np.float32) * sw, cfg.act)
        w2[g] = _store(rng.standard_normal((d, h), dtype=np.float32) * sw, cfg.act)
    return MoEInputs(cfg, _store(x, cfg.act), _store(wg, cfg.act), bias, w1, w3, w2)


def make_routing(T: int, E: int, k: int, seed: int = 1, skew: float = 0.0) -> np.ndarray:
    """Synthetic top-k expert ids [T, k] int32 with k distinct experts per token.

    skew = 0 draws uniformly; skew = s > 0 draws experts with Zipf(s)-like
    weights (expert 0 hottest), without replacement per token. Used to drive
    the dispatch and combine stages independently of the gate.
    """
    rng = np.random.default_rng(seed)
    if skew > 0:
        p = (np.arange(E, dtype=np.float64) + 1.0) ** (-skew)
    else:
        p = np.ones(E, dtype=np.float64)
    # Gumbel top-k = sampling without replacement proportional to p
    g = rng.gumbel(size=(T, E)) + np.log(p)[None, :]
    idx = np.argsort(-g, axis=1, kind="stable")[:, :k]
    return np.ascontiguousarray(idx, dtype=np.int32)


def make_rows(n: int, d: int, act: str, seed: int = 2, sigma: float = 0.5) -> np.ndarray:
    """n random rows in the activation storage dtype (synthetic expert outputs)."""
    rng = np.random.default_rng(seed)
    return _store(rng.standard_normal((n, d), dtype=np.float32) * np.float32(sigma), act)


def make_weights(T: int, k: int, seed: int = 3) -> np.ndarray:
    """Positive per-token weights [T, k] float32 summing to ~1 per token."""
    rng = np.random.default_rng(seed)
    w = rng.random((T, k), dtype=np.float32) + np.float32(0.05)
    return (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
