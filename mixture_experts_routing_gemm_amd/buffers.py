"""Device buffers for one moe_forward call (allocation plumbing only)."""

from __future__ import annotations

import torch

from ._binding import STAGE_FORWARD, alloc_workspace, moe_forward, moe_forward_traced

_ACT = {0: torch.float32, 1: torch.bfloat16}


class ForwardBuffers:
    """Outputs and workspace of moe_forward for one shape, allocated once."""

    def __init__(self, shape, device="cuda"):
        T, d, E, k = shape.T, shape.d, shape.E, shape.k
        self.shape = shape
        self.y = torch.empty((T, d), dtype=_ACT[shape.act], device=device)
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=device)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.counts = torch.empty((E,), dtype=torch.int32, device=device)
        self.offsets = torch.empty((E + 1,), dtype=torch.int32, device=device)
        self.dest_row = torch.empty((T, k), dtype=torch.int32, device=device)
        self.src_token = torch.empty((max(T * k, 1),), dtype=torch.int32, device=device)
        self.ws = alloc_workspace(shape, STAGE_FORWARD, device)

    def run(self, x, w_gate, bias, w1, w3, w2, stream=None, events=None):
        args = (self.shape, x, w_gate, bias, w1, w3, w2, self.y, self.topk_idx, self.topk_w,
                self.counts, self.offsets, self.dest_row, self.src_token, self.ws)
        if events is None:
            moe_forward(*args, stream=stream)
        else:
            moe_forward_traced(*args, events=events, stream=stream)
        return self.y
