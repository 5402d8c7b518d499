"""The largest operands the boundary accepts (GPU): 4 GiB and beyond.

K is at its maximum (32768). The GEMM's buffer-load kernels address an
operand with 32-bit offsets, so up to M x K < 2^32 they run (here at
M x K = 2^32 - 32768, their largest operand, the last row ending on the last
addressable byte), and from 2^32 on the 64-bit generic kernel takes over
(M x K = 2^32 exactly). The per-token quantizer, the calibration maxima, the
weight fold and the LoRA shrink and expand each read an 8 GiB bf16 input. Every output row listed in ROWS is compared with the
oracle bit for bit: the first and last rows, the rows on both sides of the
2^31- and 2^32-byte offsets of the INT8 operand, and the middle.
"""
import numpy as np
import pytest
import torch

import bench
import oracle.sq_oracle as O
import w8a8_smoothquant_int8_amd as sq

pytestmark = pytest.mark.gpu
F32 = np.float32
K = 32768


def rows_of(M):
    r = {0, 1, M // 2, M - 2, M - 1, (1 << 31) // K - 1, (1 << 31) // K, (1 << 32) // K - 1}
    return np.array(sorted(v for v in r if 0 <= v < M), np.int64)


def bits_equal(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("M,tile", [(131071, None), (131072, "generic")])
def test_gemm_at_4_gib_operand(M, tile):
    N = 256
    assert (M * K >= 1 << 32) == (tile == "generic")
    picked = bench.gemm_tile(M, N, K)
    assert (picked == "generic") == (tile == "generic")
    g = torch.Generator(device="cuda")
    g.manual_seed(M)
    X = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda", generator=g)
    W = torch.randint(-127, 128, (N, K), dtype=torch.int8, device="cuda", generator=g)
    a = torch.rand(M, device="cuda", generator=g) * 0.05 + 1e-3
    w = torch.rand(N, device="cuda", generator=g) * 1e-3 + 1e-5
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    sq.sq_w8a8_gemm(X, W, a, w, Y)
    torch.cuda.synchronize()
    rows = rows_of(M)
    idx = torch.from_numpy(rows).cuda()
    xq = X.index_select(0, idx).cpu().numpy()
    ref = O.dequantize(O.int8_gemm(xq, W.cpu().numpy()), a.cpu().numpy()[rows], w.cpu().numpy(),
                       "bf16")
    got = Y.index_select(0, idx).float().cpu().numpy()
    assert bits_equal(got, ref), picked
    # every row was written (the NaN fill is gone everywhere)
    assert not bool(torch.isnan(Y).any())
    del X, Y
    torch.cuda.empty_cache()


def test_quant_per_token_8_gib_input():
    M = 131072
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    X = torch.randn((M, K), dtype=torch.bfloat16, device="cuda", generator=g)
    cols = torch.randperm(K, device="cuda", generator=g)[:328]
    X[:, cols] *= 50
    X[M - 2].zero_()                                  # a zero row near the end
    s = torch.exp(torch.rand(K, device="cuda", generator=g) * 3 - 1)
    Xq = torch.full((M, K), 99, dtype=torch.int8, device="cuda")
    a = torch.full((M,), -1.0, dtype=torch.float32, device="cuda")
    sq.sq_quant_per_token(X, s, Xq, a)
    torch.cuda.synchronize()
    rows = rows_of(M)
    idx = torch.from_numpy(rows).cuda()
    x = X.index_select(0, idx).float().cpu().numpy()
    rq, ra = O.quantize_per_token(x, s.cpu().numpy())
    assert bits_equal(a.cpu().numpy()[rows], ra)
    assert bits_equal(Xq.index_select(0, idx).cpu().numpy(), rq)
    # every row was written: the sentinel code 99 is out of range and the scales are >= 0
    assert int(Xq.max()) <= 127 and float(a.min()) >= 0.0
    del X, Xq
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def big_x():
    """An 8 GiB bf16 input [131072, 32768] with outlier columns."""
    M = 131072
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    X = torch.randn((M, K), dtype=torch.bfloat16, device="cuda", generator=g)
    cols = torch.randperm(K, device="cuda", generator=g)[:328]
    X[:, cols] *= 50
    yield X, cols
    del X
    torch.cuda.empty_cache()


def test_calibrate_absmax_8_gib(big_x):
    """Column maxima over all 131072 rows, checked on a set of columns (the
    outlier ones among them) against the oracle over those whole columns."""
    X, outl = big_x
    act = torch.zeros(K, dtype=torch.float32, device="cuda")
    sq.sq_calibrate_absmax(X, act)
    cols = torch.cat([outl[:16], torch.tensor([0, 1, 8191, 8192, K - 2, K - 1], device="cuda")])
    xc = X.index_select(1, cols).float().cpu().numpy()
    ref = O.calibrate_absmax(xc)
    assert bits_equal(act.index_select(0, cols).cpu().numpy(), ref)


def test_fold_quant_weights_8_gib(big_x):
    """The 8 GiB input as a weight matrix [N = 131072, K]: codes and scales of
    the sampled rows, bit for bit."""
    W, _ = big_x
    N = W.shape[0]
    s = torch.exp(torch.rand(K, device="cuda") * 2 - 1)
    Wq = torch.full((N, K), 99, dtype=torch.int8, device="cuda")
    ws = torch.full((N,), -1.0, dtype=torch.float32, device="cuda")
    sq.sq_fold_quant_weights(W, s, Wq, ws)
    torch.cuda.synchronize()
    rows = rows_of(N)
    idx = torch.from_numpy(rows).cuda()
    rq, rs = O.fold_and_quantize_weights(W.index_select(0, idx).float().cpu().numpy(), s.cpu().numpy())
    assert bits_equal(Wq.index_select(0, idx).cpu().numpy(), rq)
    assert bits_equal(ws.cpu().numpy()[rows], rs)
    assert int(Wq.max()) <= 127 and float(ws.min()) >= 0.0
    del Wq
    torch.cuda.empty_cache()


def test_lora_apply_8_gib(big_x):
    """LoRA shrink and expand on the 8 GiB input (rank 16, N = 256), the
    sampled rows within the LoRA bar."""
    X, _ = big_x
    M = X.shape[0]
    N, r = 256, 16
    g = torch.Generator(device="cuda")
    g.manual_seed(13)
    A = (torch.randn((r, K), device="cuda", generator=g) * 0.01).to(torch.bfloat16)
    B = (torch.randn((N, r), device="cuda", generator=g) * 0.01).to(torch.bfloat16)
    Y = (torch.randn((M, N), device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    rows = rows_of(M)
    idx = torch.from_numpy(rows).cuda()
    y0 = Y.index_select(0, idx).float().cpu().numpy()
    ws = torch.empty(sq.sq_lora_workspace_bytes(M, K, r), dtype=torch.uint8, device="cuda")
    sq.sq_lora_apply(X, A, B, Y, ws)
    torch.cuda.synchronize()
    ref = O.lora_apply(y0, X.index_select(0, idx).float().cpu().numpy(), "bf16",
                       A.float().cpu().numpy(), B.float().cpu().numpy(), 1.0, "bf16")
    got = Y.index_select(0, idx).float().cpu().numpy().astype(np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.all(np.abs(got - ref) <= 2e-2 * np.abs(ref) + 2e-2 * rms)
