"""The SmoothQuant W8A8 linear path for a group of projections sharing one input.

Calibrate -> smooth and fold -> quantize the input -> INT8 GEMM with dequant per
projection -> bf16 LoRA delta per projection. Projections that read the same
input (Q/K/V, or gate/up) share one smoothing vector, because the division by
s is applied to their common input ("SmoothQuant" explainer, "How it works",
Step 5); their weights are stacked into one [sum N, K] matrix and each GEMM
runs on its row range at its own shape.

This module only sequences calls into libsq and owns the device buffers (all
allocated once, up front, so the forward pass allocates nothing and can be
captured into a HIP graph). It performs no arithmetic of its own.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Tuple

import torch

from . import (sq_calibrate_absmax, sq_lora_apply, sq_lora_apply_segmented,
               sq_lora_workspace_bytes, sq_quant_per_token, sq_smooth_fold,
               sq_static_act_scale, sq_w8a8_gemm)

_OUT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@dataclass
class SegmentedLora:
    seg_start: torch.Tensor       # int32 [S+1], device
    seg_adapter: torch.Tensor     # int32 [S], device
    A: List[torch.Tensor]         # per adapter [r_a, K] bf16
    B: List[torch.Tensor]         # per adapter [N, r_a] bf16
    ranks: torch.Tensor           # int32 [n_adapters], device
    A_ptrs: torch.Tensor          # int64 [n_adapters], device
    B_ptrs: torch.Tensor
    max_rank: int


class LinearGroup:
    """One activation input feeding one or more projections."""

    def __init__(self, W: torch.Tensor, rows: Dict[str, Tuple[int, int]], alpha: float,
                 out_dtype: str, M: int, lora: Optional[Dict[str, Tuple[torch.Tensor, torch.Tensor]]] = None,
                 seg_lora: Optional[Dict[str, SegmentedLora]] = None, lora_scale: float = 1.0):
        dev = W.device
        self.W, self.rows, self.alpha, self.M = W, rows, float(alpha), int(M)
        Ntot, K = W.shape
        self.K = K
        self.act_max = torch.zeros(K, dtype=torch.float32, device=dev)
        self.s = torch.empty(K, dtype=torch.float32, device=dev)
        self.Wq = torch.empty(Ntot, K, dtype=torch.int8, device=dev)
        self.w_scale = torch.empty(Ntot, dtype=torch.float32, device=dev)
        self.Xq = torch.empty(self.M, K, dtype=torch.int8, device=dev)
        self.a_scale = torch.empty(max(self.M, 1), dtype=torch.float32, device=dev)
        self.static_scale = torch.empty(1, dtype=torch.float32, device=dev)
        self.Y = {p: torch.empty(self.M, r1 - r0, dtype=_OUT[out_dtype], device=dev)
                  for p, (r0, r1) in rows.items()}
        self.lora = lora or {}
        self.seg_lora = seg_lora or {}
        self.lora_scale = float(lora_scale)
        ranks = [a.shape[0] for a, _ in self.lora.values()] + [s.max_rank for s in self.seg_lora.values()]
        wsb = sq_lora_workspace_bytes(self.M, K, max(ranks)) if ranks and self.M else 0
        self.ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)

    # -- offline ------------------------------------------------------------
    def calibrate(self, X_cal: torch.Tensor, reset: bool = True) -> None:
        if reset:
            self.act_max.zero_()
        sq_calibrate_absmax(X_cal, self.act_max)

    def fold(self) -> None:
        sq_smooth_fold(self.act_max, self.W, self.alpha, self.s, self.Wq, self.w_scale)
        sq_static_act_scale(self.act_max, self.s, self.static_scale)

    # -- per batch ----------------------------------------------------------
    def quantize(self, X: torch.Tensor, mode: str = "dynamic") -> None:
        a = self.a_scale if mode == "dynamic" else self.static_scale
        sq_quant_per_token(X, self.s, self.Xq, a, mode=mode)

    def gemm(self, proj: str, mode: str = "dynamic") -> torch.Tensor:
        r0, r1 = self.rows[proj]
        a = self.a_scale if mode == "dynamic" else self.static_scale
        sq_w8a8_gemm(self.Xq, self.Wq[r0:r1], a, self.w_scale[r0:r1], self.Y[proj], mode=mode)
        return self.Y[proj]

    def apply_lora(self, proj: str, X: torch.Tensor) -> None:
        if proj in self.lora:
            A, B = self.lora[proj]
            sq_lora_apply(X, A, B, self.Y[proj], self.ws, scale=self.lora_scale)
        elif proj in self.seg_lora:
            g = self.seg_lora[proj]
            sq_lora_apply_segmented(X, g.seg_start, g.seg_adapter, g.A_ptrs, g.B_ptrs, g.ranks,
                                    g.max_rank, self.Y[proj], self.ws, scale=self.lora_scale)

    def forward(self, X: torch.Tensor, mode: str = "dynamic") -> Dict[str, torch.Tensor]:
        self.quantize(X, mode)
        for p in self.rows:
            self.gemm(p, mode)
            self.apply_lora(p, X)
        return self.Y
