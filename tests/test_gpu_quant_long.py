"""The long-row quantizer (16-bit inputs, 16384 < K <= 32768) vs the oracle (GPU).

One block per row, persistent over the rows with the raw row double-buffered,
so the shapes cover: rows beyond one pass of the grid (the second buffer and
the row loop's odd tail), K a multiple of 4096 (every lane chunk in the row)
and ragged K (chunks past the row end, re-read and masked), zero rows, and all
four kinds (fold, per-token, static, static with the clip counter). Each
result must equal the oracle's bit for bit, and equal the block-per-row-group
kernel the library used before for these K (selected with SQ_QUANT_LONG=0).
"""
import os

import numpy as np
import pytest
import torch

import oracle.sq_oracle as O
import w8a8_smoothquant_int8_amd as sq
from synth.workloads import cast_to

pytestmark = pytest.mark.gpu
F32 = np.float32

# (rows, K): K / 8 / 512 = 4.004 .. 8 lane chunks, rows up to about 3 grid passes
SHAPES = [(37, 16400), (600, 20480), (300, 24592), (513, 28672), (19, 32768)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    assert sq.sq_query_support(0), "device 0 is not gfx950"


def rows_with_outliers(rng, M, K, dtype, sigma=1.0, factor=50.0):
    x = (rng.standard_normal((M, K)) * sigma).astype(F32)
    cols = rng.choice(K, size=max(1, K // 300), replace=False)
    x[:, cols] *= factor
    if M > 3:
        x[3] = 0.0
    t = cast_to(x, dtype)
    return t.cuda(), t.float().numpy()


def earlier_kernel(fn):
    """Run fn with the block-per-row-group kernel selected for long rows."""
    old = os.environ.get("SQ_QUANT_LONG")
    os.environ["SQ_QUANT_LONG"] = "0"
    try:
        return fn()
    finally:
        if old is None:
            del os.environ["SQ_QUANT_LONG"]
        else:
            os.environ["SQ_QUANT_LONG"] = old


def same(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,K", SHAPES)
def test_fold_long(dtype, M, K):
    rng = np.random.default_rng(11 * M + K)
    w, wn = rows_with_outliers(rng, M, K, dtype, sigma=0.02, factor=1.0)
    s = np.exp(rng.uniform(-2, 3, K)).astype(F32)
    sd = torch.from_numpy(s).cuda()

    def run():
        Wq = torch.empty(M, K, dtype=torch.int8, device="cuda")
        ws = torch.empty(M, dtype=torch.float32, device="cuda")
        sq.sq_fold_quant_weights(w, sd, Wq, ws)
        return Wq.cpu().numpy(), ws.cpu().numpy()

    Wq, ws = run()
    rq, rs = O.fold_and_quantize_weights(wn, s)
    assert same(ws, rs) and same(Wq, rq)
    Wq0, ws0 = earlier_kernel(run)
    assert same(Wq0, Wq) and same(ws0, ws)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("smooth", [True, False])
def test_per_token_long(dtype, M, K, smooth):
    rng = np.random.default_rng(13 * M + K + smooth)
    x, xn = rows_with_outliers(rng, M, K, dtype)
    s = np.exp(rng.uniform(-1, 2, K)).astype(F32) if smooth else None
    sd = torch.from_numpy(s).cuda() if smooth else None

    def run():
        Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
        a = torch.empty(M, dtype=torch.float32, device="cuda")
        sq.sq_quant_per_token(x, sd, Xq, a)
        return Xq.cpu().numpy(), a.cpu().numpy()

    Xq, a = run()
    rq, ra = O.quantize_per_token(xn, s)
    assert same(a, ra) and same(Xq, rq)
    Xq0, a0 = earlier_kernel(run)
    assert same(Xq0, Xq) and same(a0, a)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,K", SHAPES)
def test_static_and_clip_count_long(dtype, M, K):
    rng = np.random.default_rng(17 * M + K)
    xc, xcn = rows_with_outliers(rng, 64, K, dtype)
    s = np.exp(rng.uniform(-1, 2, K)).astype(F32)
    a = O.static_activation_scale(O.calibrate_absmax(xcn), s)
    # a batch three times wider than the calibration batch: many codes clip
    x, xn = rows_with_outliers(rng, M, K, dtype, sigma=3.0)
    sd = torch.from_numpy(s).cuda()
    ad = torch.tensor([a], dtype=torch.float32, device="cuda")

    def run():
        Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
        sq.sq_quant_per_token(x, sd, Xq, ad, mode="static")
        Xc = torch.empty(M, K, dtype=torch.int8, device="cuda")
        counter = torch.zeros(1, dtype=torch.int64, device="cuda")
        sq.sq_quant_static_clipped(x, sd, ad, Xc, counter)
        return Xq.cpu().numpy(), Xc.cpu().numpy(), int(counter.item())

    Xq, Xc, n = run()
    rq, clipped = O.quantize_per_tensor_static(xn, s, a)
    assert clipped > 0
    assert same(Xq, rq) and same(Xc, rq)
    assert n == clipped
    Xq0, Xc0, n0 = earlier_kernel(run)
    assert same(Xq0, Xq) and same(Xc0, Xc) and n0 == n
