"""The SmoothQuant W8A8 linear path for a group of projections sharing one input.

Calibrate -> smooth and fold -> quantize the input -> INT8 GEMM with dequant ->
bf16 LoRA delta. Projections that read the same input (Q/K/V, or gate/up)
share one smoothing vector, because the division by s is applied to their
common input ("SmoothQuant" explainer, "How it works", Step 5); their weights
are stacked into one [sum N, K] matrix.

Forward pass (fused, the default): one quantization of the input, one LoRA
shrink with every projection's A stacked along the rank (X is read once for
all adapters), and one GEMM over the stacked weights whose epilogue adds the
LoRA delta. quantize_and_shrink() does the first two in one kernel that reads
X once (sq_quant_shrink). The stacked B is block-diagonal (projection p's rows carry its B
in its own rank columns and zeros elsewhere), so each output column gets only
its own adapter's delta, exactly as separate per-projection calls would give.
Per-projection outputs are column views of one [M, sum N] buffer.

run() issues calibrate, fold and the fused forward pass of a group as one
native call (sq_linear_group_run): the same kernels, one host call.

Unfused (fuse=False): one GEMM and one shrink+expand LoRA call per
projection, the path the fused one is checked against. Per-request
(segmented) adapters always use the separate segmented call on the column
views.

This module only sequences calls into libsq and owns the device buffers (all
allocated once, up front, so the forward pass allocates nothing and can be
captured into a HIP graph). It performs no arithmetic of its own.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Tuple

import torch

from . import (SQ_GROUP_CALIBRATE, SQ_GROUP_FOLD, SQ_GROUP_FORWARD, SQ_MAX_LORA_PARTS,
               SQ_MAX_LORA_RANK,
               sq_alpha_sweep, sq_alpha_sweep_workspace_bytes, sq_calibrate_absmax,
               sq_fold_norm_weight, sq_norm_quant, sq_quant_shrink, SQError, SQ_ERR_INVALID_ARG,
               SQ_ERR_UNSUPPORTED_DTYPE, sq_linear_group_desc, sq_linear_group_run, sq_lora_apply,
               sq_lora_apply_segmented, sq_lora_shrink, sq_lora_workspace_bytes,
               sq_quant_per_token, sq_quant_static_clipped, sq_smooth_fold, sq_static_act_scale,
               sq_w8a8_gemm, sq_w8a8_gemm_lora, sq_w8a8_gemm_workspace_bytes, sq_w8a8_gemm_ws)

ALL_PHASES = SQ_GROUP_CALIBRATE | SQ_GROUP_FOLD | SQ_GROUP_FORWARD

# Largest share of clipped activation codes the static range check accepts:
# a few clipped values per million are harmless ("SmoothQuant" explainer,
# "Calibration in practice"); read here as at most 5 per million.
MAX_CLIP_RATE = 5e-6

_OUT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def alpha_sweep(X: torch.Tensor, W: torch.Tensor, alphas, mode: str = "dynamic",
                stream=None) -> dict:
    """Output error of the quantized layer against the unquantized one for each
    alpha, on the calibration batch X ("SmoothQuant" explainer, "Calibration in
    practice"): one native call, which also forms the relative errors and
    picks the best alpha, then one read of its results. Returns err (sum of
    squared errors), ref (sum of squared outputs), rel = err / ref, and best
    (the alpha of the smallest rel, the first on ties)."""
    M, K = X.shape
    ws = torch.empty(max(sq_alpha_sweep_workspace_bytes(M, W.shape[0], K), 256),
                     dtype=torch.uint8, device=X.device)
    out = torch.empty(len(alphas), 2, dtype=torch.float64, device=X.device)
    rel = torch.empty(len(alphas), dtype=torch.float64, device=X.device)
    best = torch.empty(1, dtype=torch.int32, device=X.device)
    sq_alpha_sweep(X, W, alphas, out, ws, mode=mode, rel=rel, best=best, stream=stream)
    host, rel_h, ib = out.cpu(), rel.cpu().tolist(), int(best.cpu()[0])
    return {"err": host[:, 0].tolist(), "ref": float(host[0, 1]), "rel": rel_h,
            "best": float(alphas[ib])}


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
                 seg_lora: Optional[Dict[str, SegmentedLora]] = None, lora_scale: float = 1.0,
                 fuse: bool = True, modes: Tuple[str, ...] = ("dynamic",)):
        dev = W.device
        self.W, self.rows, self.alpha, self.M = W, rows, float(alpha), int(M)
        self.modes = tuple(modes)   # activation modes this group will run
        Ntot, K = W.shape
        self.K, self.Ntot = K, Ntot
        self.act_max = torch.zeros(K, dtype=torch.float32, device=dev)
        self.s = torch.empty(K, dtype=torch.float32, device=dev)
        self.Wq = torch.empty(Ntot, K, dtype=torch.int8, device=dev)
        self.w_scale = torch.empty(Ntot, dtype=torch.float32, device=dev)
        self.Xq = torch.empty(self.M, K, dtype=torch.int8, device=dev)
        self.a_scale = torch.empty(max(self.M, 1), dtype=torch.float32, device=dev)
        self.static_scale = torch.empty(1, dtype=torch.float32, device=dev)
        self.clip_count = torch.zeros(1, dtype=torch.int64, device=dev)   # static mode
        self.clip_elems = 0                                                # elements counted
        self.Yg = torch.empty(self.M, Ntot, dtype=_OUT[out_dtype], device=dev)
        self.Y = {p: self.Yg[:, r0:r1] for p, (r0, r1) in rows.items()}
        self.lora = lora or {}
        self.seg_lora = seg_lora or {}
        self.lora_scale = float(lora_scale)

        # Stacked LoRA for the fused path: every projection has an adapter and
        # the total rank fits one call.
        r_tot = sum(a.shape[0] for a, _ in self.lora.values())
        self.fused = bool(fuse and self.lora and set(self.lora) == set(rows)
                          and r_tot <= SQ_MAX_LORA_RANK)
        self.lora_parts = None
        if self.fused:
            order = sorted(rows, key=lambda p: rows[p][0])     # adapters stacked in column order
            self.A_stack = torch.cat([self.lora[p][0] for p in order], dim=0).contiguous()
            self.B_blk = torch.zeros(Ntot, r_tot, dtype=torch.bfloat16, device=dev)
            c, parts, n_prev = 0, [], 0
            for p in order:
                A, B = self.lora[p]
                r0, r1 = rows[p]
                self.B_blk[r0:r1, c:c + A.shape[0]] = B
                c += A.shape[0]
                parts.append((r1, c) if r0 == n_prev else None)
                n_prev = r1
            # The projection table lets the GEMM epilogue skip the zero blocks of
            # B_blk; it needs the projections to tile the columns in order.
            if (len(parts) > 1 and None not in parts and n_prev == Ntot
                    and len(parts) <= SQ_MAX_LORA_PARTS):
                self.lora_parts = parts
            self.T = torch.empty(self.M, r_tot, dtype=torch.bfloat16, device=dev)
        ranks = ([r_tot] if self.fused else [a.shape[0] for a, _ in self.lora.values()]) + \
                [s.max_rank for s in self.seg_lora.values()]
        wsb = sq_lora_workspace_bytes(self.M, K, max(ranks)) if ranks and self.M else 0
        # decode-sized GEMMs without LoRA split K across blocks in the same workspace
        self.gemm_ws_bytes = sq_w8a8_gemm_workspace_bytes(self.M, Ntot, K) if self.M else 0
        self.ws = torch.empty(max(wsb, self.gemm_ws_bytes, 16), dtype=torch.uint8, device=dev)

    # -- offline ------------------------------------------------------------
    def calibrate(self, X_cal: torch.Tensor, reset: bool = True) -> None:
        if reset:
            self.act_max.zero_()
        sq_calibrate_absmax(X_cal, self.act_max)

    def choose_alpha(self, X_cal: torch.Tensor, alphas, mode: str = "dynamic") -> dict:
        """Set this group's alpha to the sweep's best over `alphas` on X_cal
        (over all the group's projections at once: they share one s)."""
        r = alpha_sweep(X_cal, self.W, alphas, mode)
        self.alpha = r["best"]
        self._desc_key = None            # the native-call descriptor carries alpha
        return r

    def fold(self) -> None:
        sq_smooth_fold(self.act_max, self.W, self.alpha, self.s, self.Wq, self.w_scale)
        if "static" in self.modes:
            sq_static_act_scale(self.act_max, self.s, self.static_scale)

    # -- the normalization in front of the group ----------------------------
    def set_norm(self, gamma: torch.Tensor, beta: Optional[torch.Tensor] = None,
                 kind: str = "rms", eps: float = 1e-5) -> None:
        """The RMSNorm / LayerNorm that produces this group's input. After
        fold(), fold_norm() divides its weight and bias by s ("SmoothQuant"
        explainer, "How it works", Step 5), and forward_norm() runs the group
        straight from the residual stream."""
        self.norm = (gamma, beta, kind, float(eps))
        K = self.K
        self.norm_g = torch.empty(K, dtype=torch.float32, device=gamma.device)
        self.norm_b = torch.empty(K, dtype=torch.float32, device=gamma.device) \
            if beta is not None else None

    def fold_norm(self) -> None:
        gamma, beta, _, _ = self.norm
        sq_fold_norm_weight(gamma, beta, self.s, self.norm_g, self.norm_b)

    def quantize_norm(self, H: torch.Tensor, mode: str = "dynamic") -> None:
        _, _, kind, eps = self.norm
        sq_norm_quant(H, kind, self.norm_g, self.norm_b, eps, self.Xq, self._a(mode), mode=mode)

    def forward_norm(self, H: torch.Tensor, mode: str = "dynamic") -> Dict[str, torch.Tensor]:
        """norm -> (folded) smoothing -> quant in one kernel, then the GEMM. The
        LoRA path reads the unsmoothed norm output, which this kernel does not
        write, so groups with adapters use forward() on the norm output."""
        if self.lora or self.seg_lora:
            raise ValueError("forward_norm covers groups without LoRA adapters")
        self.quantize_norm(H, mode)
        self.gemm_all(mode)
        return self.Y

    # -- per batch ----------------------------------------------------------
    def _a(self, mode: str) -> torch.Tensor:
        return self.a_scale if mode == "dynamic" else self.static_scale

    def quantize(self, X: torch.Tensor, mode: str = "dynamic", count_clips: bool = False) -> None:
        """count_clips (static mode): also add the number of clamped codes to
        clip_count (device counter, kept across calls until reset_clips)."""
        if mode == "static" and count_clips:
            sq_quant_static_clipped(X, self.s, self.static_scale, self.Xq, self.clip_count)
            self.clip_elems += X.shape[0] * X.shape[1]
        else:
            sq_quant_per_token(X, self.s, self.Xq, self._a(mode), mode=mode)

    def reset_clips(self) -> None:
        self.clip_count.zero_()
        self.clip_elems = 0

    def clip_rate(self) -> float:
        """Share of clipped codes over the static batches counted so far (reads
        the device counter: synchronises with the stream)."""
        return int(self.clip_count.item()) / self.clip_elems if self.clip_elems else 0.0

    def gemm(self, proj: str, mode: str = "dynamic") -> torch.Tensor:
        """One projection's GEMM without LoRA."""
        r0, r1 = self.rows[proj]
        sq_w8a8_gemm(self.Xq, self.Wq[r0:r1], self._a(mode), self.w_scale[r0:r1], self.Y[proj],
                     mode=mode)
        return self.Y[proj]

    def gemm_all(self, mode: str = "dynamic") -> None:
        """All projections' GEMMs as one call over the stacked weights, without LoRA
        (with the split-K workspace where the shape uses one)."""
        sq_w8a8_gemm_ws(self.Xq, self.Wq, self._a(mode), self.w_scale, self.Yg,
                        self.ws if self.gemm_ws_bytes else None, mode=mode)

    def lora_shrink(self, X: torch.Tensor) -> None:
        sq_lora_shrink(X, self.A_stack, self.T, self.ws)

    def quantize_and_shrink(self, X: torch.Tensor, mode: str = "dynamic") -> None:
        """The quant and the stacked LoRA shrink: one kernel reading X once where
        sq_quant_shrink takes the shape (16-bit X, K within its register budget),
        else the two separate calls."""
        if getattr(self, "_qs_ok", True):
            try:
                sq_quant_shrink(X, self.s, self.Xq, self._a(mode), self.A_stack, self.T, mode=mode)
                self._qs_ok = True
                return
            except SQError as e:          # rejected on the host: nothing was enqueued
                if e.status not in (SQ_ERR_INVALID_ARG, SQ_ERR_UNSUPPORTED_DTYPE):
                    raise
                self._qs_ok = False
        self.quantize(X, mode)
        self.lora_shrink(X)

    def gemm_all_lora(self, mode: str = "dynamic") -> None:
        """All projections' GEMMs as one call, each adding its LoRA delta in the epilogue."""
        sq_w8a8_gemm_lora(self.Xq, self.Wq, self._a(mode), self.w_scale, self.T, self.B_blk,
                          self.Yg, scale=self.lora_scale, mode=mode)

    def apply_lora(self, proj: str, X: torch.Tensor, stream=None) -> None:
        """One projection's LoRA delta as a separate shrink + expand call."""
        if proj in self.lora:
            A, B = self.lora[proj]
            sq_lora_apply(X, A, B, self.Y[proj], self.ws, scale=self.lora_scale, stream=stream)
        elif proj in self.seg_lora:
            g = self.seg_lora[proj]
            sq_lora_apply_segmented(X, g.seg_start, g.seg_adapter, g.A_ptrs, g.B_ptrs, g.ranks,
                                    g.max_rank, self.Y[proj], self.ws, scale=self.lora_scale,
                                    stream=stream)

    # -- one native call per step ---------------------------------------------
    def run(self, X: torch.Tensor, X_cal: Optional[torch.Tensor], flags: int = ALL_PHASES,
            mode: str = "dynamic", stream=None, events=None, seg_events=None) -> None:
        """The selected phases (calibrate, fold, forward) as one sq_linear_group_run
        call: the same kernels as calibrate() + fold() + forward() on the fused
        path, launched from native code. Groups with per-request (segmented)
        adapters then issue each projection's segmented LoRA call on the same
        stream, as forward() does. Not for unstacked single adapters.
        events: None or sq_group_events(...) for the group call; seg_events:
        None or a (begin, end) pair of torch events around the segmented calls."""
        if self.lora and not self.fused:
            raise ValueError("run() covers the stacked-LoRA (fused), segmented and no-LoRA groups")
        key = (X.data_ptr(), None if X_cal is None else X_cal.data_ptr(), mode)
        if getattr(self, "_desc_key", None) != key:
            lora = dict(A=self.A_stack, B=self.B_blk, T=self.T, lora_scale=self.lora_scale,
                        lora_parts=self.lora_parts) if self.fused else {}
            self._desc = sq_linear_group_desc(X, X_cal, self.W, self.alpha, mode, self.act_max,
                                              self.s, self.Wq, self.w_scale, self.Xq, self._a(mode),
                                              self.Yg, workspace=self.ws, **lora)
            self._desc_inputs = (X, X_cal)      # keep the tensors the pointers refer to alive
            self._desc_key = key
        sq_linear_group_run(self._desc, flags, stream, events)
        if self.seg_lora and (flags & SQ_GROUP_FORWARD) and self.M > 0:
            st = stream if stream is not None else torch.cuda.current_stream()
            if seg_events is not None:
                seg_events[0].record(st)
            for p in self.seg_lora:
                self.apply_lora(p, X, stream=st)
            if seg_events is not None:
                seg_events[1].record(st)

    def forward_static_checked(self, X: torch.Tensor, max_rate: float = MAX_CLIP_RATE
                               ) -> Tuple[Dict[str, torch.Tensor], float, bool]:
        """Static-scale forward pass with a range check: the batch is quantized
        with the calibrated per-tensor scale while its clipped codes are
        counted; if their share exceeds max_rate the scale no longer covers the
        batch and the pass is redone with per-token dynamic scales (the more
        robust variant; "SmoothQuant" explainer, "Calibration in practice").
        Returns (outputs, clip rate of this batch, fell_back). Reads the
        counter on the host, so it synchronises once per call."""
        base, elems = self.clip_count.clone(), X.shape[0] * X.shape[1]
        Y = self.forward(X, "static", count_clips=True)
        rate = (int(self.clip_count.item()) - int(base.item())) / elems if elems else 0.0
        if rate > max_rate:
            return self.forward(X, "dynamic"), rate, True
        return Y, rate, False

    def forward(self, X: torch.Tensor, mode: str = "dynamic",
                count_clips: bool = False) -> Dict[str, torch.Tensor]:
        self.quantize(X, mode, count_clips)
        if self.fused:
            self.lora_shrink(X)
            self.gemm_all_lora(mode)
        elif self.lora:
            for p in self.rows:
                self.gemm(p, mode)
                self.apply_lora(p, X)
        else:
            self.gemm_all(mode)
            for p in self.seg_lora:
                self.apply_lora(p, X)
        return self.Y
