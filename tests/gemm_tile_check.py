"""GEMM parity under one tile configuration, run as a child process by
test_gpu_gemm_tiles.py with SQ_GEMM_TILE set (the library reads the override
once per process). Shapes are ragged against every tile size and cover one,
two, three and eight 128-byte K-tiles, so the pipelined kernel's prologue and
its last-K-tile paths all run; LoRA ranks cover one and two 64-rank passes
(the second full or partial) and a scale other than 1. Bars as in test_gpu_parity.py: INT32 and dequantized
outputs bit-exact, LoRA outputs within the LoRA bar. Prints one JSON line and
exits non-zero on any failure."""
import json
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import oracle.sq_oracle as O  # noqa: E402
import w8a8_smoothquant_int8_amd as sq  # noqa: E402
from synth.workloads import cast_to  # noqa: E402

F32 = np.float32
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
SHAPES = [(300, 400, 128), (300, 400, 256), (257, 448, 384), (513, 1040, 1024), (64, 208, 512),
          (1, 48, 128), (17, 400, 1024), (33, 1040, 384), (64, 5120, 2560)]


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t, out):
    t = t.cpu()
    return t.float().numpy() if out != "f16" else t.numpy()


def bits_equal(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def lora_ok(got, ref, out):
    g, r = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(r ** 2))
    if not np.all(np.abs(g - r) <= 2e-2 * np.abs(r) + 2e-2 * rms):
        return False
    return out == "f32" or np.mean(np.asarray(got) != np.asarray(ref)) < 0.01


def main():
    failures, n = [], 0
    for (M, N, K) in SHAPES:
        rng = np.random.default_rng(M * 7 + N * 3 + K)
        xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
        wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
        acc_ref = O.int8_gemm(xq, wq)
        dx, dw = dev(xq), dev(wq)
        acc = torch.empty(M, N, dtype=torch.int32, device="cuda")
        sq.sq_w8a8_gemm_i32(dx, dw, acc)
        n += 1
        if not np.array_equal(acc.cpu().numpy(), acc_ref):
            failures.append(f"i32 {M}x{N}x{K}")
        a_dyn = rng.uniform(1e-3, 5e-2, M).astype(F32)
        a_st = rng.uniform(1e-3, 5e-2, 1).astype(F32)
        w = rng.uniform(1e-5, 1e-3, N).astype(F32)
        for out, mode in [("bf16", "dynamic"), ("f16", "static"), ("f32", "dynamic")]:
            a = a_dyn if mode == "dynamic" else a_st
            Y = torch.zeros(M, N, dtype=DT[out], device="cuda")
            sq.sq_w8a8_gemm(dx, dw, dev(a), dev(w), Y, mode=mode)
            ref = O.dequantize(acc_ref, a if mode == "dynamic" else a[0], w, out)
            n += 1
            if not bits_equal(host(Y, out), ref):
                failures.append(f"dequant {out} {mode} {M}x{N}x{K}")
        for r, scale, out, mode in [(48, 1.0, "bf16", "dynamic"), (128, 1.0, "f16", "static"),
                                    (72, 1.0, "bf16", "dynamic"), (24, 0.5, "f32", "dynamic"),
                                    (16, 1.0, "f32", "static")]:
            a = a_dyn if mode == "dynamic" else a_st
            t = cast_to(rng.normal(0, 0.5, (M, r)).astype(F32), "bf16")
            b = cast_to(rng.normal(0, 0.05, (N, r)).astype(F32), "bf16")
            Y = torch.zeros(M, N, dtype=DT[out], device="cuda")
            sq.sq_w8a8_gemm_lora(dx, dw, dev(a), dev(w), t.cuda(), b.cuda(), Y, scale=scale, mode=mode)
            y = O.dequantize(acc_ref, a if mode == "dynamic" else a[0], w, out)
            ref = O.lora_expand_add(y, t.float().numpy(), b.float().numpy(), scale, out)
            n += 1
            if not lora_ok(host(Y, out), ref, out):
                failures.append(f"lora r{r} scale{scale} {out} {mode} {M}x{N}x{K}")
    print(json.dumps({"tile": os.environ.get("SQ_GEMM_TILE", "auto"), "cases": n, "failures": failures}),
          flush=True)
    return 1 if failures else 0


if __name__ == "__main__":
    sys.exit(main())
