"""The largest operands the boundary accepts (GPU): 4 GiB and beyond.

K is at its maximum (32768). The GEMM's buffer-load kernels address an
operand with 32-bit offsets, so up to M x K < 2^32 they run (here at
M x K = 2^32 - 32768, their largest operand, the last row ending on the last
addressable byte), and from 2^32 on the 64-bit generic kernel takes over
(M x K = 2^32 exactly). The per-token quantizer reads an 8 GiB input and
writes a 4 GiB output. Every output row listed in ROWS is compared with the
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
