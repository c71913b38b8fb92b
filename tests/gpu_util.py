"""Helpers for the GPU parity tests: host <-> device copies and error norms."""

from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

HAVE_GPU = torch.cuda.is_available()

# oracle worker threads for full-size checks (at most 16 host threads)
ORACLE_THREADS = min(16, os.cpu_count() or 1)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> contiguous CUDA tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """CUDA tensor -> numpy; bf16 comes back as uint16 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def rel_l2(got, ref) -> float:
    got = as_f64(np.asarray(got))
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


class RowErrors:
    """Relative L2 over a whole tensor, accumulated chunk by chunk, and the
    worst single row's relative L2."""

    def __init__(self):
        self.num = 0.0
        self.den = 0.0
        self.worst = 0.0
        self.worst_row = -1
        self.rows = 0

    def add(self, got, ref, row0=0):
        g = as_f64(np.asarray(got))
        r = np.asarray(ref, dtype=np.float64)
        dn = np.sum((g - r) ** 2, axis=1)
        rn = np.sum(r ** 2, axis=1)
        self.num += float(dn.sum())
        self.den += float(rn.sum())
        per = np.sqrt(dn / np.where(rn > 0, rn, 1.0))
        i = int(np.argmax(per))
        if per[i] > self.worst:
            self.worst, self.worst_row = float(per[i]), row0 + i
        self.rows += len(r)

    @property
    def rel(self):
        return float(np.sqrt(self.num / self.den)) if self.den > 0 else float(np.sqrt(self.num))

    def check(self, what, tol):
        say(f"{what}: rel-L2 {self.rel:.3e} over {self.rows} rows, worst row {self.worst_row} "
            f"{self.worst:.3e} (bound {tol:.0e})")
        assert self.rows > 0
        assert self.rel <= tol, f"{what}: rel-L2 {self.rel:.3e} > {tol}"
        assert self.worst <= tol, f"{what}: row {self.worst_row} rel-L2 {self.worst:.3e} > {tol}"


def act_torch(act: str):
    return torch.float32 if act == "f32" else torch.bfloat16


requires_gpu = pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")
