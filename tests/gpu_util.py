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


def act_torch(act: str):
    return torch.float32 if act == "f32" else torch.bfloat16


requires_gpu = pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")
