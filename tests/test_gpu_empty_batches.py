"""M = 0 through every entry point that takes a row count (GPU).

The boundary's rule is that an empty batch is a no-op that returns SQ_OK:
no kernel runs and no output is written. Each call here goes through the C
ABI with real (non-null) buffers, since torch gives empty tensors a null
pointer, and every output buffer starts filled with a sentinel that must
survive the call.
"""
import ctypes

import pytest
import torch

import w8a8_smoothquant_int8_amd as sq

pytestmark = pytest.mark.gpu

K, N, R = 256, 128, 16


def P(t):
    return ctypes.c_void_p(t.data_ptr())


@pytest.fixture()
def bufs():
    d = "cuda"
    b = {
        "X": torch.ones(4, K, dtype=torch.bfloat16, device=d),
        "s": torch.ones(K, dtype=torch.float32, device=d),
        "Xq": torch.full((4, K), 7, dtype=torch.int8, device=d),
        "a": torch.full((4,), 3.0, dtype=torch.float32, device=d),
        "Wq": torch.ones(N, K, dtype=torch.int8, device=d),
        "w": torch.ones(N, dtype=torch.float32, device=d),
        "Y": torch.full((4, N), 1.5, dtype=torch.bfloat16, device=d),
        "acc": torch.full((4, N), 11, dtype=torch.int32, device=d),
        "A": torch.ones(R, K, dtype=torch.bfloat16, device=d),
        "B": torch.ones(N, R, dtype=torch.bfloat16, device=d),
        "T": torch.full((4, R), 2.0, dtype=torch.bfloat16, device=d),
        "g": torch.ones(K, dtype=torch.float32, device=d),
        "stats": torch.full((4, 2), 5.0, dtype=torch.float32, device=d),
        "ws": torch.zeros(1 << 20, dtype=torch.uint8, device=d),
        "seg_start": torch.zeros(2, dtype=torch.int32, device=d),
        "seg_adapter": torch.zeros(1, dtype=torch.int32, device=d),
        "ranks": torch.full((1,), R, dtype=torch.int32, device=d),
    }
    b["A_ptrs"] = sq.pointer_table([b["A"]], "cuda")
    b["B_ptrs"] = sq.pointer_table([b["B"]], "cuda")
    before = {k: v.clone() for k, v in b.items()}
    yield b
    torch.cuda.synchronize()
    for k, v in b.items():
        assert torch.equal(v, before[k]), f"{k} changed by an empty batch"


def test_quant_per_token_empty(bufs):
    b = bufs
    assert sq.lib().sq_quant_per_token(P(b["X"]), sq.SQ_BF16, 0, K, K, P(b["s"]),
                                       sq.SQ_ACT_PER_TOKEN_DYNAMIC, P(b["Xq"]), P(b["a"]),
                                       None) == sq.SQ_OK


def test_norm_quant_empty(bufs):
    b = bufs
    assert sq.lib().sq_norm_quant(P(b["X"]), sq.SQ_BF16, 0, K, K, sq.SQ_NORM["rms"], P(b["g"]),
                                  None, 1e-5, sq.SQ_ACT_PER_TOKEN_DYNAMIC, P(b["Xq"]), P(b["a"]),
                                  P(b["stats"]), None) == sq.SQ_OK


def test_quant_shrink_empty(bufs):
    b = bufs
    assert sq.lib().sq_quant_shrink(P(b["X"]), sq.SQ_BF16, 0, K, K, P(b["s"]),
                                    sq.SQ_ACT_PER_TOKEN_DYNAMIC, P(b["Xq"]), P(b["a"]), P(b["A"]),
                                    R, P(b["T"]), R, None) == sq.SQ_OK


@pytest.mark.parametrize("call", ["gemm", "gemm_ws", "gemm_i32", "gemm_lora"])
def test_gemm_empty(bufs, call):
    b = bufs
    L = sq.lib()
    mode = sq.SQ_ACT_PER_TOKEN_DYNAMIC
    if call == "gemm":
        rc = L.sq_w8a8_gemm(P(b["Xq"]), P(b["Wq"]), P(b["a"]), mode, P(b["w"]), 0, N, K, P(b["Y"]),
                            sq.SQ_BF16, N, None)
    elif call == "gemm_ws":
        rc = L.sq_w8a8_gemm_ws(P(b["Xq"]), P(b["Wq"]), P(b["a"]), mode, P(b["w"]), 0, N, K,
                               P(b["Y"]), sq.SQ_BF16, N, P(b["ws"]), b["ws"].numel(), None)
    elif call == "gemm_i32":
        rc = L.sq_w8a8_gemm_i32(P(b["Xq"]), P(b["Wq"]), 0, N, K, P(b["acc"]), None)
    else:
        rc = L.sq_w8a8_gemm_lora(P(b["Xq"]), P(b["Wq"]), P(b["a"]), mode, P(b["w"]), 0, N, K,
                                 P(b["T"]), R, P(b["B"]), R, 1.0, P(b["Y"]), sq.SQ_BF16, N, None)
    assert rc == sq.SQ_OK


def test_lora_shrink_and_apply_empty(bufs):
    b = bufs
    L = sq.lib()
    assert L.sq_lora_shrink(P(b["X"]), sq.SQ_BF16, 0, K, K, P(b["A"]), R, P(b["T"]), R,
                            P(b["ws"]), b["ws"].numel(), None) == sq.SQ_OK
    assert L.sq_lora_apply(P(b["X"]), sq.SQ_BF16, 0, K, K, P(b["A"]), P(b["B"]), R, 1.0,
                           P(b["Y"]), sq.SQ_BF16, N, N, P(b["ws"]), b["ws"].numel(),
                           None) == sq.SQ_OK


@pytest.mark.parametrize("noalloc", [False, True])
def test_lora_segmented_empty_batch(bufs, noalloc):
    """M_total = 0 with one (empty) request [0, 0) that names a real adapter."""
    b = bufs
    L = sq.lib()
    args = (P(b["X"]), sq.SQ_BF16, 0, K, K, 1, P(b["seg_start"]), P(b["seg_adapter"]), 1,
            P(b["A_ptrs"]), P(b["B_ptrs"]), P(b["ranks"]), R, 1.0, P(b["Y"]), sq.SQ_BF16, N, N)
    if noalloc:
        rc = L.sq_lora_apply_segmented_noalloc(*args, None)
    else:
        rc = L.sq_lora_apply_segmented(*args, P(b["ws"]), b["ws"].numel(), None)
    assert rc == sq.SQ_OK
