"""Seeded synthetic workloads for the SmoothQuant W8A8 linear path.

This module draws random tensors and nothing else. It holds none of the
method's arithmetic (no scales, no quantization, no products), so both the
CPU oracle's tests and the HIP path's tests and benchmark can take their
inputs from it without sharing any computation.

Structure of the inputs. The SmoothQuant explainer ("Why activations are
harder than weights") describes activations where a few channels run one to
two orders of magnitude above the others, and do so at the same channel
positions for every token. Each activation input below is therefore N(0, 1)
with a fixed set of outlier columns multiplied by per-column factors. Weights
are N(0, 0.02); LoRA factors are N(0, 0.01) in bf16. A calibration batch for
an input is an independent draw with the same outlier columns and factors
("How it works", Step 4, the calibration statistics), min(M, 512) rows.

Randomness. Every tensor has its own numpy PCG64 stream, derived from
SeedSequence(entropy=seed, spawn_key=key) with a fixed integer key per tensor
role, so a tensor does not depend on which other tensors were drawn first.
"""
from __future__ import annotations

import dataclasses
import math
import zlib
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

_TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def cast_to(x32: np.ndarray, dtype: str) -> torch.Tensor:
    """Cast an fp32 numpy array to a CPU torch tensor of the workload dtype (RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(_TORCH_DTYPES[dtype])


def _key(*parts) -> Tuple[int, ...]:
    out = []
    for p in parts:
        if isinstance(p, str):
            out.append(zlib.crc32(p.encode()) & 0x7FFFFFFF)
        else:
            out.append(int(p))
    return tuple(out)


def rng_for(seed: int, *parts) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=_key(*parts)))


@dataclasses.dataclass(frozen=True)
class Projection:
    name: str
    input: str   # which activation input feeds it
    N: int       # output features


@dataclasses.dataclass(frozen=True)
class Outliers:
    kind: str                 # "count_fixed": n columns x factor; "frac_fixed"; "frac_loguniform"
    count: int = 0
    frac: float = 0.0
    factor: float = 1.0
    lo: float = 1.0
    hi: float = 1.0

    def n_cols(self, K: int) -> int:
        if self.kind == "count_fixed":
            return self.count
        return int(round(self.frac * K))


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    description: str
    M: int
    dtype: str                    # activation / weight dtype: f32, f16, bf16
    out_dtype: str                # GEMM output dtype
    alpha: float
    inputs: Tuple[Tuple[str, int], ...]          # (input name, K)
    projections: Tuple[Projection, ...]
    outliers: Outliers
    lora_rank: int = 0            # single adapter per projection (0 = none)
    act_modes: Tuple[str, ...] = ("dynamic",)
    segmented: Optional[dict] = None             # multi-tenant LoRA description

    # ---- shapes -------------------------------------------------------------
    def K_of(self, inp: str) -> int:
        return dict(self.inputs)[inp]

    def group(self, inp: str) -> List[Projection]:
        """Projections sharing one input (and so one smoothing vector)."""
        return [p for p in self.projections if p.input == inp]

    def group_rows(self, inp: str) -> Dict[str, Tuple[int, int]]:
        """Row range [r0, r1) of each projection inside the group's stacked weight."""
        out, r = {}, 0
        for p in self.group(inp):
            out[p.name] = (r, r + p.N)
            r += p.N
        return out

    def calib_rows(self) -> int:
        return min(self.M, 512)

    def gemm_ops(self) -> int:
        return sum(2 * self.M * p.N * self.K_of(p.input) for p in self.projections)

    # ---- tensors ------------------------------------------------------------
    def outlier_columns(self, inp: str, seed: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        K = self.K_of(inp)
        n = self.outliers.n_cols(K)
        rng = rng_for(seed, self.name, inp, "outliers")
        cols = np.sort(rng.choice(K, size=n, replace=False))
        if self.outliers.kind == "frac_loguniform":
            f = np.exp(rng.uniform(math.log(self.outliers.lo), math.log(self.outliers.hi), size=n))
        else:
            f = np.full(n, self.outliers.factor)
        return cols, f.astype(np.float32)

    def _acts(self, inp: str, rows: int, role: str, seed: int) -> torch.Tensor:
        K = self.K_of(inp)
        x = rng_for(seed, self.name, inp, role).standard_normal((rows, K), dtype=np.float32)
        cols, f = self.outlier_columns(inp, seed)
        x[:, cols] *= f[None, :]
        return cast_to(x, self.dtype)

    def x(self, inp: str, seed: int = 0) -> torch.Tensor:
        """Activation input [M, K] in the workload dtype."""
        return self._acts(inp, self.M, "x", seed)

    def x_cal(self, inp: str, seed: int = 0) -> torch.Tensor:
        """Calibration batch [min(M,512), K]: independent rows, same outlier columns."""
        return self._acts(inp, self.calib_rows(), "cal", seed)

    def w(self, proj: str, seed: int = 0) -> torch.Tensor:
        p = next(q for q in self.projections if q.name == proj)
        K = self.K_of(p.input)
        w = rng_for(seed, self.name, proj, "w").normal(0.0, 0.02, size=(p.N, K)).astype(np.float32)
        return cast_to(w, self.dtype)

    def w_group(self, inp: str, seed: int = 0) -> torch.Tensor:
        """Stacked weight [sum N, K] of the projections fed by `inp` (nn.Linear [out, in])."""
        return torch.cat([self.w(p.name, seed) for p in self.group(inp)], dim=0)

    def lora(self, proj: str, rank: Optional[int] = None, seed: int = 0,
             adapter: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
        """LoRA factors A [r, K] and B [N, r] in bf16, N(0, 0.01)."""
        p = next(q for q in self.projections if q.name == proj)
        r = self.lora_rank if rank is None else rank
        K = self.K_of(p.input)
        rng = rng_for(seed, self.name, proj, "lora", adapter)
        a = rng.normal(0.0, 0.01, size=(r, K)).astype(np.float32)
        b = rng.normal(0.0, 0.01, size=(p.N, r)).astype(np.float32)
        return cast_to(a, "bf16"), cast_to(b, "bf16")

    # ---- multi-tenant segments ---------------------------------------------
    def segments(self, seed: int = 0) -> Dict[str, np.ndarray]:
        """Request lengths, segment starts, adapter per request and rank per adapter.

        Lengths are drawn uniformly from [lo, hi] and repaired to sum to M:
        scale by M / sum, round, clamp to [lo, hi], then add or remove one
        token on seeded random requests until the sum is exact.
        """
        sp = self.segmented
        assert sp is not None
        rng = rng_for(seed, self.name, "segments")
        n, lo, hi = sp["requests"], sp["len_lo"], sp["len_hi"]
        L = rng.integers(lo, hi + 1, size=n).astype(np.int64)
        L = np.clip(np.rint(L * (self.M / L.sum())), lo, hi).astype(np.int64)
        while L.sum() != self.M:
            i = int(rng.integers(0, n))
            if L.sum() > self.M and L[i] > lo:
                L[i] -= 1
            elif L.sum() < self.M and L[i] < hi:
                L[i] += 1
        seg_start = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
        seg_adapter = rng.integers(0, sp["adapters"], size=n).astype(np.int32)
        ranks = rng.choice(np.asarray(sp["ranks"]), size=sp["adapters"]).astype(np.int32)
        return {"lengths": L, "seg_start": seg_start, "seg_adapter": seg_adapter, "ranks": ranks}


_LLAMA3_8B_OUT = Outliers("frac_loguniform", frac=0.01, lo=20.0, hi=100.0)

WORKLOADS: Dict[str, Workload] = {}


def _reg(w: Workload) -> None:
    WORKLOADS[w.name] = w


_reg(Workload(
    name="tiny_m16_k256_n256",
    description="Tiny single linear: M=16, K=N=256, fp32 activations with 4 outlier "
                "channels x50, alpha 0.5, LoRA rank 8, bf16 output",
    M=16, dtype="f32", out_dtype="bf16", alpha=0.5,
    inputs=(("x", 256),),
    projections=(Projection("linear", "x", 256),),
    outliers=Outliers("count_fixed", count=4, factor=50.0),
    lora_rank=8,
))

_reg(Workload(
    name="llama3_8b_proj_m2048",
    description="Llama-3-8B-shaped projections, bf16, M=2048: Q/O 4096->4096, K/V 4096->1024, "
                "gate/up 4096->14336, down 14336->4096; 1% outlier channels x20-100 "
                "(log-uniform); alpha 0.5; LoRA rank 16 on every projection",
    M=2048, dtype="bf16", out_dtype="bf16", alpha=0.5,
    inputs=(("attn_in", 4096), ("o_in", 4096), ("mlp_in", 4096), ("down_in", 14336)),
    projections=(Projection("q", "attn_in", 4096), Projection("k", "attn_in", 1024),
                 Projection("v", "attn_in", 1024), Projection("o", "o_in", 4096),
                 Projection("gate", "mlp_in", 14336), Projection("up", "mlp_in", 14336),
                 Projection("down", "down_in", 4096)),
    outliers=_LLAMA3_8B_OUT, lora_rank=16,
))

for _m, _tag in ((64, "decode_m64"), (4096, "prefill_m4096")):
    _reg(Workload(
        name=f"opt13b_layer_{_tag}",
        description=f"OPT-13B-shaped layer, fp16, M={_m}: q/k/v/o 5120->5120, fc1 5120->20480, "
                    "fc2 20480->5120; 0.5% outlier channels x60; alpha 0.8; per-token dynamic "
                    "and per-tensor static activation scales; no LoRA",
        M=_m, dtype="f16", out_dtype="f16", alpha=0.8,
        inputs=(("attn_in", 5120), ("o_in", 5120), ("fc1_in", 5120), ("fc2_in", 20480)),
        projections=(Projection("q", "attn_in", 5120), Projection("k", "attn_in", 5120),
                     Projection("v", "attn_in", 5120), Projection("o", "o_in", 5120),
                     Projection("fc1", "fc1_in", 20480), Projection("fc2", "fc2_in", 5120)),
        outliers=Outliers("frac_fixed", frac=0.005, factor=60.0),
        act_modes=("dynamic", "static"),
    ))

_reg(Workload(
    name="multitenant_lora_m8192",
    description="Multi-tenant LoRA on Llama-3-8B shapes: 8192 tokens in 64 requests "
                "(lengths 32-256), 32 bf16 adapters with ranks in {8,16,64}, on Q/K/V/O",
    M=8192, dtype="bf16", out_dtype="bf16", alpha=0.5,
    inputs=(("attn_in", 4096), ("o_in", 4096)),
    projections=(Projection("q", "attn_in", 4096), Projection("k", "attn_in", 1024),
                 Projection("v", "attn_in", 1024), Projection("o", "o_in", 4096)),
    outliers=_LLAMA3_8B_OUT,
    segmented={"requests": 64, "len_lo": 32, "len_hi": 256, "adapters": 32, "ranks": (8, 16, 64)},
))

_reg(Workload(
    name="llama2_70b_mlp_m8192",
    description="Llama-2-70B-shaped MLP block, bf16, M=8192: gate/up 8192->28672, "
                "down 28672->8192; 1% outlier channels x20-100; alpha 0.5; LoRA rank 64",
    M=8192, dtype="bf16", out_dtype="bf16", alpha=0.5,
    inputs=(("mlp_in", 8192), ("down_in", 28672)),
    projections=(Projection("gate", "mlp_in", 28672), Projection("up", "mlp_in", 28672),
                 Projection("down", "down_in", 8192)),
    outliers=_LLAMA3_8B_OUT, lora_rank=64,
))


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def ragged(M: int, K: int, N: int, dtype: str = "bf16", out_dtype: str = "bf16",
           alpha: float = 0.5, lora_rank: int = 0, n_out: int = 3, factor: float = 40.0,
           name: Optional[str] = None) -> Workload:
    """A one-projection workload of arbitrary shape, for tile-edge and ragged-tail tests."""
    return Workload(
        name=name or f"ragged_m{M}_k{K}_n{N}_{dtype}",
        description="ragged test shape", M=M, dtype=dtype, out_dtype=out_dtype, alpha=alpha,
        inputs=(("x", K),), projections=(Projection("linear", "x", N),),
        outliers=Outliers("count_fixed", count=min(n_out, K), factor=factor),
        lora_rank=lora_rank,
    )


def sample_rows(M: int, n_every: int = 64, extra: Sequence[int] = ()) -> np.ndarray:
    """Deterministic row subset: first, last, every n-th, plus given rows."""
    rows = set(range(0, M, n_every)) | {0, M - 1} | {int(r) for r in extra if 0 <= r < M}
    return np.array(sorted(rows), dtype=np.int64)
