"""Device-resident MoE layer on top of the C ABI.

torch provides the device memory (weights, workspace, outputs) and the stream;
every step of the forward pass runs in libmoe.so through `moe_forward`.
"""
from __future__ import annotations

import numpy as np

from . import (MoEProblem, moe_aux_loss, moe_bias_update, moe_forward, moe_workspace_size,
               problem)
from .configs import MoEConfig


def to_device(a: np.ndarray, dtype: str, device="cuda"):
    """Host array (float32, or bf16 bit patterns as uint16) -> torch tensor."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    return t.to(device)


def to_host(t, dtype: str) -> np.ndarray:
    """torch tensor -> float32 array, or uint16 bit patterns for bf16."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class MoELayer:
    """One MoE layer with its weights resident in HBM."""

    def __init__(self, T: int, d: int, E: int, K: int, F: int, dtype: str, w_router, w1, w3, w2,
                 capacity: int = -1, device="cuda", flags: int = 0):
        import torch
        self.T, self.d, self.E, self.K, self.F = T, d, E, K, F
        self.dtype = dtype
        self.capacity = capacity
        self.device = device
        self.w_router, self.w1, self.w3, self.w2 = w_router, w1, w3, w2
        self.torch_dtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.flags = flags
        self.p: MoEProblem = problem(T, d, E, K, F, dtype, capacity, flags)
        self.ws = torch.empty(moe_workspace_size(self.p), dtype=torch.uint8, device=device)

    @classmethod
    def from_host(cls, cfg: MoEConfig, inputs: dict, device="cuda", T: int | None = None,
                  flags: int = 0):
        dt = cfg.dtype
        return cls(cfg.T if T is None else T, cfg.d, cfg.E, cfg.K, cfg.F, dt,
                   to_device(inputs["w_router"], dt, device), to_device(inputs["w1"], dt, device),
                   to_device(inputs["w3"], dt, device), to_device(inputs["w2"], dt, device),
                   cfg.capacity, device, flags)

    def alloc_debug(self, losses: bool = False) -> dict:
        """Device buffers for every optional output of moe_forward; with
        losses, also the two router regularisers (z_loss, aux_topk)."""
        import torch
        T, E, K = self.T, self.E, self.K
        dev = self.device
        f32, i32 = torch.float32, torch.int32
        extra = {}
        if losses:
            extra = {"z_loss": torch.full((1,), -1.0, dtype=f32, device=dev),
                     "aux_topk": torch.full((1,), -1.0, dtype=f32, device=dev)}
        return extra | {
            "logits": torch.empty((T, E), dtype=f32, device=dev),
            "probs": torch.empty((T, E), dtype=f32, device=dev),
            "prob_sum": torch.empty((E,), dtype=f32, device=dev),
            "topk_ids": torch.empty((T, K), dtype=i32, device=dev),
            "topk_w": torch.empty((T, K), dtype=f32, device=dev),
            "counts": torch.empty((E,), dtype=i32, device=dev),
            "kept": torch.empty((E,), dtype=i32, device=dev),
            "offsets": torch.empty((E + 1,), dtype=i32, device=dev),
            "assign_row": torch.empty((T * K,), dtype=i32, device=dev),
            "row_assign": torch.empty((T * K,), dtype=i32, device=dev),
        }

    def forward(self, x, logit_bias=None, y=None, dbg: dict | None = None, stream=None):
        import torch
        if y is None:
            y = torch.empty((self.T, self.d), dtype=self.torch_dtype, device=self.device)
        moe_forward(self.p, x, self.w_router, self.w1, self.w3, self.w2, logit_bias, y, self.ws,
                    dbg, stream)
        return y

    def aux_loss(self, counts, prob_sum, out=None, stream=None):
        import torch
        if out is None:
            out = torch.empty((1,), dtype=torch.float32, device=self.device)
        moe_aux_loss(self.p, counts, prob_sum, out, stream)
        return out

    def bias_update(self, counts, alpha: float, bias, stream=None):
        moe_bias_update(self.p, counts, alpha, bias, stream)
        return bias
