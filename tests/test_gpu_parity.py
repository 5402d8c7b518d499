"""HIP path vs the CPU oracle, stage by stage, on the same seeded inputs (GPU).

Bars: INT8 codes, INT32 accumulators, maxima, scales: bit-exact. Dequantized
bf16/fp16/fp32 outputs: bit-exact (the kernels use the oracle's operation
order; the stated tolerance of 1 ulp / 1e-3 is not needed). LoRA-added
outputs: |gpu - oracle| <= 2e-2 |oracle| + 2e-2 rms(oracle) elementwise.
Every stage gets the oracle's inputs for that stage, so a difference upstream
cannot cascade.
"""
import numpy as np
import pytest
import torch

import oracle.sq_oracle as O
import w8a8_smoothquant_int8_amd as sq
from synth.workloads import cast_to

pytestmark = pytest.mark.gpu
F32 = np.float32
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    assert sq.sq_query_support(0), "device 0 is not gfx950"
    torch.manual_seed(0)


def npf(t):
    return t.detach().float().cpu().numpy()


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x)) if isinstance(x, np.ndarray) else x
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def acts(rng, M, K, dtype, n_out=3, factor=50.0, ld=None, sigma=1.0):
    """Random N(0, sigma) matrix with outlier columns, as a (possibly strided) device tensor,
    and its exact fp32 values."""
    x = (rng.standard_normal((M, K)) * sigma).astype(F32)
    cols = rng.choice(K, size=min(n_out, K), replace=False)
    x[:, cols] *= factor
    t = cast_to(x, dtype)
    if ld is not None and ld > K:
        wide = torch.zeros(M, ld, dtype=t.dtype)
        wide[:, :K] = t
        return wide.cuda()[:, :K], t.float().numpy()
    return t.cuda(), t.float().numpy()


def bits_equal(a, b):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


# ---------------------------------------------------------------------------
# Calibration absmax
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("M,K,ld", [(1, 16, 16), (37, 272, 288), (300, 1040, 1040), (2048, 4096, 4096)])
def test_calibrate_absmax(dtype, M, K, ld):
    rng = np.random.default_rng(M * 7 + K)
    x1, x1n = acts(rng, M, K, dtype, ld=ld)
    x2, x2n = acts(rng, max(M // 2, 1), K, dtype, factor=80.0)
    am = torch.zeros(K, dtype=torch.float32, device="cuda")
    sq.sq_calibrate_absmax(x1, am)
    sq.sq_calibrate_absmax(x2, am)
    ref = O.calibrate_absmax(x2n, O.calibrate_absmax(x1n))
    assert bits_equal(npf(am), ref)


# ---------------------------------------------------------------------------
# Smoothing scale
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("alpha", [0.5, 0.8, 0.0, 1.0, 0.3])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_smooth_scale(alpha, dtype):
    rng = np.random.default_rng(11)
    K, N = 4096, 640
    am = np.exp(rng.uniform(np.log(0.3), np.log(400), K)).astype(F32)
    am[:3] = 0.0                                    # dead channels hit the 1e-5 clamp
    w = cast_to(rng.normal(0, 0.02, (N, K)).astype(F32), dtype)
    s = torch.empty(K, dtype=torch.float32, device="cuda")
    sq.sq_smooth_scale(dev(am), w.cuda(), alpha, s)
    ref = O.smoothing_scale(am, O.weight_absmax(w.float().numpy()), alpha)
    got = npf(s)
    if alpha in (0.5, 0.0, 1.0):
        assert bits_equal(got, ref)                 # sqrt / exact-power forms
    else:
        # fp64 pow on both sides, one rounding to fp32: agree except when the
        # exact value straddles an fp32 rounding boundary; never beyond 1 ulp.
        ulps = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
        assert ulps.max() <= 1 and np.count_nonzero(ulps) <= 2, np.count_nonzero(ulps)


# ---------------------------------------------------------------------------
# Fold + per-output-channel weight quantization
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("N,K,ld", [(1, 16, 16), (16, 272, 288), (300, 4096, 4096), (33, 14336, 14336),
                                    (2100, 14336, 14336), (257, 8192, 8208), (24, 28672, 28672),
                                    (40, 20480, 20480), (17, 5120, 5136)])
def test_fold_quant_weights(dtype, N, K, ld):
    rng = np.random.default_rng(N + K)
    w, wn = acts(rng, N, K, dtype, n_out=0, ld=ld, sigma=0.02)
    if N > 2:
        w[1].zero_()
        wn[1] = 0.0
    s = np.exp(rng.uniform(-2, 3, K)).astype(F32)
    Wq = torch.empty(N, K, dtype=torch.int8, device="cuda")
    ws = torch.empty(N, dtype=torch.float32, device="cuda")
    sq.sq_fold_quant_weights(w, dev(s), Wq, ws)
    rq, rs = O.fold_and_quantize_weights(wn, s)
    assert bits_equal(npf(ws), rs)
    assert bits_equal(Wq.cpu().numpy(), rq)


# ---------------------------------------------------------------------------
# Activation quantization (smoothing divide + per-token / per-tensor)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("M,K,ld", [(1, 16, 16), (5, 48, 64), (300, 256, 256), (130, 4096, 4112),
                                    (64, 5120, 5120), (257, 8192, 8208), (70, 14336, 14336),
                                    (2100, 14336, 14336), (9, 20480, 20480), (40, 28672, 28672)])
@pytest.mark.parametrize("smooth", [True, False])
def test_quant_dynamic(dtype, M, K, ld, smooth):
    rng = np.random.default_rng(M * 3 + K)
    x, xn = acts(rng, M, K, dtype, ld=ld)
    if M > 3:
        x[2].zero_()
        xn[2] = 0.0
    s = np.exp(rng.uniform(-1, 2, K)).astype(F32) if smooth else None
    Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    a = torch.empty(M, dtype=torch.float32, device="cuda")
    sq.sq_quant_per_token(x, dev(s) if smooth else None, Xq, a)
    rq, ra = O.quantize_per_token(xn, s)
    assert bits_equal(npf(a), ra)
    assert bits_equal(Xq.cpu().numpy(), rq)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,K", [(7, 272), (256, 5120), (64, 20480)])
def test_quant_static_with_clipping(dtype, M, K):
    rng = np.random.default_rng(5 + K)
    xc, xcn = acts(rng, 64, K, dtype, factor=60.0)
    x, xn = acts(rng, M, K, dtype, factor=60.0)
    x[0, 0] = 1e3                                   # beyond the calibrated range: clips
    xn[0, 0] = x[0, 0].float().item()
    s = np.exp(rng.uniform(-1, 2, K)).astype(F32)
    am = torch.zeros(K, dtype=torch.float32, device="cuda")
    sq.sq_calibrate_absmax(xc, am)
    a = torch.empty(1, dtype=torch.float32, device="cuda")
    sq.sq_static_act_scale(am, dev(s), a)
    ra = O.static_activation_scale(O.calibrate_absmax(xcn), s)
    assert npf(a)[0] == ra
    Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    sq.sq_quant_per_token(x, dev(s), Xq, a, mode="static")
    rq, clipped = O.quantize_per_tensor_static(xn, s, ra)
    assert clipped >= 1
    assert bits_equal(Xq.cpu().numpy(), rq)


def test_quant_division_vectors_and_ties():
    # [2.25, 1.125] -> [127, 63] and [3.75, 1.875] -> [127, 64] (IEEE division,
    # half to even), padded to K = 16; and the hand-worked 4x4 example's ties.
    x = np.zeros((2, 16), F32)
    x[0, :2] = [2.25, 1.125]
    x[1, :2] = [3.75, 1.875]
    Xq = torch.empty(2, 16, dtype=torch.int8, device="cuda")
    a = torch.empty(2, dtype=torch.float32, device="cuda")
    sq.sq_quant_per_token(dev(x), None, Xq, a)
    assert Xq.cpu().numpy()[:, :2].tolist() == [[127, 63], [127, 64]]
    X44 = np.zeros((4, 16), F32)
    X44[:, :4] = [[254, 0.3125, -1.75, 0.03125], [-256, 4, 3, -0.5], [64, -1, 16, 1],
                  [-32, 0.5, -1, 0.75]]
    s = np.ones(16, F32)
    s[:4] = [32, 2, 8, 1]
    Xq = torch.empty(4, 16, dtype=torch.int8, device="cuda")
    a = torch.empty(4, dtype=torch.float32, device="cuda")
    sq.sq_quant_per_token(dev(X44), dev(s), Xq, a)
    assert Xq.cpu().numpy()[:, :4].tolist() == [[127, 2, -4, 0], [-127, 32, 6, -8],
                                                 [127, -32, 127, 64], [-127, 32, -16, 95]]


@pytest.mark.parametrize("K,per_row", [(256, 1), (4096, 3), (14336, 2), (20480, 1)])
def test_quant_smoothing_division_near_midpoints(K, per_row):
    """x / s on quotients within about 2^-48 of an fp32 rounding midpoint (the
    cases an approximate division rounds the wrong way first). Each row holds
    per_row such quotients, the largest one alone setting the row max, so the
    row's a_scale = fp32(fp32(x / s) / 127) exposes any error in fp32(x / s);
    a_scale and the codes must be bit-exact. K spans the wave-per-row and the
    block-per-row quantizers."""
    from div_cases import near_midpoint_pairs
    M = min(1024, K // per_row)              # every pair gets a channel of its own
    xs, ds, _r = near_midpoint_pairs(M * per_row, K + per_row, exp_range=0)   # x / s in [0.5, 1)
    s = np.exp(np.random.default_rng(K).uniform(-1, 1, K)).astype(F32)
    x = np.zeros((M, K), F32)
    cols = np.random.default_rng(K + 7).permutation(K)[:M * per_row].reshape(M, per_row)
    for i in range(M):
        for t in range(per_row):
            c = cols[i, t]
            s[c] = ds[i * per_row + t]
            # 4^-t keeps the first pair the row max (quotients below 0.25 for t >= 1)
            x[i, c] = np.ldexp(xs[i * per_row + t], -2 * t)
    Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    a = torch.empty(M, dtype=torch.float32, device="cuda")
    sq.sq_quant_per_token(dev(x), dev(s), Xq, a)
    rq, ra = O.quantize_per_token(x, s)
    assert bits_equal(npf(a), ra)
    assert bits_equal(Xq.cpu().numpy(), rq)


# ---------------------------------------------------------------------------
# INT8 GEMM
# ---------------------------------------------------------------------------
GEMM_SHAPES = [(1, 16, 16), (17, 48, 80), (130, 272, 400), (300, 144, 1040), (257, 1024, 4096),
               (64, 5120, 5120), (129, 384, 14336)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_i32(M, N, K):
    rng = np.random.default_rng(M + N + K)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    acc = torch.empty(M, N, dtype=torch.int32, device="cuda")
    sq.sq_w8a8_gemm_i32(dev(xq), dev(wq), acc)
    assert np.array_equal(acc.cpu().numpy(), O.int8_gemm(xq, wq))


def test_gemm_i32_extreme_magnitude():
    K = 28672
    xq = np.full((40, K), 127, np.int8)
    xq[1::2] = -127
    wq = np.full((48, K), 127, np.int8)
    wq[::3, ::2] = -127
    acc = torch.empty(40, 48, dtype=torch.int32, device="cuda")
    sq.sq_w8a8_gemm_i32(dev(xq), dev(wq), acc)
    ref = O.int8_gemm(xq, wq)
    assert ref.max() == K * 127 * 127
    assert np.array_equal(acc.cpu().numpy(), ref)


# Decode shapes whose K is split across blocks with a workspace (M = 64, 48,
# 40, 33 and 17; 2, 3, 4, 8 and 19 slices; a ragged last 64-column block at
# N = 1040 and N = 208, whose second 32-column tile lies past N; the last slice
# shorter than the others at K = 20480, 5120, 20352), plus shapes that take no
# workspace (128 or more column blocks of 64; K too short for two slices of
# 8 K-tiles): bit-exact against the oracle and the unsplit call.
@pytest.mark.parametrize("out", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("mode", ["dynamic", "static"])
@pytest.mark.parametrize("M,N,K,split", [(64, 5120, 20480, True), (17, 1040, 8192, True),
                                         (40, 208, 20352, True), (64, 20480, 5120, False),
                                         (64, 5120, 5120, True), (64, 8192, 8192, False),
                                         (64, 2048, 1920, False), (1, 16400, 2048, False),
                                         (64, 5120, 2048, True), (33, 6144, 3072, True),
                                         (48, 4096, 8192, True)])
def test_gemm_ws_split_k(out, mode, M, N, K, split):
    """Workspace GEMM against the plain one and the oracle, bit for bit; the
    split shapes take 2 (64x5120x2048, 33x6144x3072), 3 (64x5120x20480,
    64x5120x5120), 4 (48x4096x8192), 8 (17x1040x8192) and 19 (40x208x20352)
    K slices."""
    rng = np.random.default_rng(M + N + K)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    a = rng.uniform(1e-3, 5e-2, M if mode == "dynamic" else 1).astype(F32)
    w = rng.uniform(1e-5, 1e-3, N).astype(F32)
    need = sq.sq_w8a8_gemm_workspace_bytes(M, N, K)
    assert (need > 0) == split
    ws = torch.full((max(need, 16),), 0x5A, dtype=torch.uint8, device="cuda") if need else None
    X, W, A, Wsc = dev(xq), dev(wq), dev(a), dev(w)
    Y1 = torch.zeros(M, N, dtype=DT[out], device="cuda")
    Y2 = torch.zeros(M, N, dtype=DT[out], device="cuda")
    for _ in range(2):   # the second call finds the first call's partial sums in the workspace
        sq.sq_w8a8_gemm_ws(X, W, A, Wsc, Y1, ws, mode=mode)
    sq.sq_w8a8_gemm(X, W, A, Wsc, Y2, mode=mode)
    assert torch.equal(Y1.view(torch.uint8), Y2.view(torch.uint8))
    ref = O.dequantize(O.int8_gemm(xq, wq), a if mode == "dynamic" else a[0], w, out)
    got = Y1.cpu()
    got = got.float().numpy() if out != "f16" else got.numpy()
    assert bits_equal(got, ref)


@pytest.mark.parametrize("out", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("mode", ["dynamic", "static"])
# (64, 20480, 5120) and (33, 16448, 1024): decode shapes with more 64-column
# blocks than CUs, run in 128-column blocks (the second with a half-empty last one)
@pytest.mark.parametrize("M,N,K", [(33, 48, 272), (300, 1024, 4096), (64, 20480, 5120),
                                   (33, 16448, 1024)])
def test_gemm_dequant(out, mode, M, N, K):
    rng = np.random.default_rng(M * N + K)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    a = rng.uniform(1e-3, 5e-2, M if mode == "dynamic" else 1).astype(F32)
    w = rng.uniform(1e-5, 1e-3, N).astype(F32)
    ldy = N + (16 if N < 1000 else 0)
    Yw = torch.zeros(M, ldy, dtype=DT[out], device="cuda")
    Y = Yw[:, :N]
    sq.sq_w8a8_gemm(dev(xq), dev(wq), dev(a), dev(w), Y, mode=mode)
    ref = O.dequantize(O.int8_gemm(xq, wq), a if mode == "dynamic" else a[0], w, out)
    got = Y.cpu()
    got = got.float().numpy() if out != "f16" else got.numpy()
    assert bits_equal(got, ref)


# ---------------------------------------------------------------------------
# LoRA
# ---------------------------------------------------------------------------
def lora_close(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    err = np.abs(got - ref)
    ok = err <= 2e-2 * np.abs(ref) + 2e-2 * rms
    return bool(ok.all()), float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))


def lora_inputs(rng, M, K, N, r, xdt, ydt):
    x, xn = acts(rng, M, K, xdt, factor=20.0)
    a = cast_to(rng.normal(0, 0.01, (r, K)).astype(F32), "bf16")
    b = cast_to(rng.normal(0, 0.01, (N, r)).astype(F32), "bf16")
    y = cast_to(rng.normal(0, 0.5, (M, N)).astype(F32), ydt)
    return x, xn, a, b, y


# ranks 40, 72 and 128: the expand's rank steps of 32 (2, 3, 4; T zero-padded
# past r), the 128-rank shrink chunking, and fp32 Y with four rank steps
@pytest.mark.parametrize("r", [8, 16, 40, 64, 72, 128])
@pytest.mark.parametrize("xdt,ydt", [("bf16", "bf16"), ("f32", "bf16"), ("f16", "f16"), ("bf16", "f32")])
@pytest.mark.parametrize("M,K,N", [(1, 16, 16), (33, 272, 144), (300, 4096, 1024), (70, 14336, 64)])
def test_lora_apply(r, xdt, ydt, M, K, N):
    rng = np.random.default_rng(r + M + K + N)
    x, xn, a, b, y = lora_inputs(rng, M, K, N, r, xdt, ydt)
    Y = y.cuda()
    ws = torch.empty(sq.sq_lora_workspace_bytes(M, K, r), dtype=torch.uint8, device="cuda")
    sq.sq_lora_apply(x, a.cuda(), b.cuda(), Y, ws, scale=1.0)
    yn = y.float().numpy() if ydt != "f16" else y.numpy()
    ref = O.lora_apply(yn, xn, xdt, a.float().numpy(), b.float().numpy(), 1.0, ydt)
    ok, rel = lora_close(Y.cpu().float().numpy(), ref)
    assert ok, rel


def test_lora_zero_b_leaves_output_bitwise():
    rng = np.random.default_rng(3)
    x, xn, a, b, y = lora_inputs(rng, 64, 512, 256, 16, "bf16", "bf16")
    Y = y.cuda()
    ws = torch.empty(sq.sq_lora_workspace_bytes(64, 512, 16), dtype=torch.uint8, device="cuda")
    sq.sq_lora_apply(x, a.cuda(), torch.zeros_like(b).cuda(), Y, ws)
    assert torch.equal(Y.cpu(), y)


def make_segments(rng, M, n_adapters, ranks, with_none=True):
    cuts = np.sort(rng.choice(np.arange(1, M), size=min(M - 1, 9), replace=False))
    seg_start = np.concatenate([[0], cuts, [M]]).astype(np.int32)
    S = len(seg_start) - 1
    seg_adapter = rng.integers(0, n_adapters, S).astype(np.int32)
    if with_none:
        seg_adapter[rng.integers(0, S)] = -1
    return seg_start, seg_adapter


@pytest.mark.parametrize("M,K,N", [(97, 272, 144), (700, 4096, 1024)])
@pytest.mark.parametrize("ydt", ["bf16", "f32"])
def test_lora_segmented(M, K, N, ydt):
    rng = np.random.default_rng(M + K)
    ranks = [8, 16, 64, 16]
    x, xn = acts(rng, M, K, "bf16", factor=20.0)
    As = [cast_to(rng.normal(0, 0.01, (r, K)).astype(F32), "bf16") for r in ranks]
    Bs = [cast_to(rng.normal(0, 0.01, (N, r)).astype(F32), "bf16") for r in ranks]
    seg_start, seg_adapter = make_segments(rng, M, len(ranks), ranks)
    y = cast_to(rng.normal(0, 0.5, (M, N)).astype(F32), ydt)
    Ad = [t.cuda() for t in As]
    Bd = [t.cuda() for t in Bs]
    Y = y.cuda()
    ws = torch.empty(sq.sq_lora_workspace_bytes(M, K, 64), dtype=torch.uint8, device="cuda")
    sq.sq_lora_apply_segmented(x, dev(seg_start), dev(seg_adapter), sq.pointer_table(Ad, "cuda"),
                               sq.pointer_table(Bd, "cuda"), dev(np.array(ranks, np.int32)), 64, Y, ws)
    ref = O.lora_apply_segmented(y.float().numpy(), xn, "bf16", seg_start, seg_adapter,
                                 [t.float().numpy() for t in As], [t.float().numpy() for t in Bs],
                                 1.0, ydt)
    got = Y.cpu().float().numpy()
    ok, rel = lora_close(got, ref)
    assert ok, rel
    for g in np.nonzero(seg_adapter < 0)[0]:        # requests without adapter: untouched
        r0, r1 = seg_start[g], seg_start[g + 1]
        assert torch.equal(Y[r0:r1].cpu(), y[r0:r1])


@pytest.mark.parametrize("xdt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("ranks", [[8, 24, 64, 16], [128, 8, 40]])
def test_lora_segmented_short_and_empty_requests(xdt, ranks):
    """Many requests per 64-row block (lengths 0-5 among longer ones), empty
    requests, requests without adapter, ranks that are not a multiple of 16,
    and K not a multiple of the 256-element chunk."""
    rng = np.random.default_rng(len(ranks) * 7 + len(xdt))
    M, K, N = 333, 528, 208
    lens = []
    while sum(lens) < M:
        lens.append(int(rng.integers(0, 6)) if rng.random() < 0.7 else int(rng.integers(20, 90)))
    lens[-1] -= sum(lens) - M
    seg_start = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    nseg = len(lens)
    seg_adapter = rng.integers(0, len(ranks), nseg).astype(np.int32)
    seg_adapter[rng.random(nseg) < 0.15] = -1
    x, xn = acts(rng, M, K, xdt, factor=20.0)
    As = [cast_to(rng.normal(0, 0.01, (r, K)).astype(F32), "bf16") for r in ranks]
    Bs = [cast_to(rng.normal(0, 0.01, (N, r)).astype(F32), "bf16") for r in ranks]
    y = cast_to(rng.normal(0, 0.5, (M, N)).astype(F32), "bf16")
    Ad = [t.cuda() for t in As]
    Bd = [t.cuda() for t in Bs]
    Y = y.cuda()
    mr = max(ranks)
    ws = torch.empty(sq.sq_lora_workspace_bytes(M, K, mr), dtype=torch.uint8, device="cuda")
    sq.sq_lora_apply_segmented(x, dev(seg_start), dev(seg_adapter), sq.pointer_table(Ad, "cuda"),
                               sq.pointer_table(Bd, "cuda"), dev(np.array(ranks, np.int32)), mr, Y, ws)
    ref = O.lora_apply_segmented(y.float().numpy(), xn, xdt, seg_start, seg_adapter,
                                 [t.float().numpy() for t in As], [t.float().numpy() for t in Bs],
                                 1.0, "bf16")
    ok, rel = lora_close(Y.cpu().float().numpy(), ref)
    assert ok, rel
    for g in np.nonzero(seg_adapter < 0)[0]:
        r0, r1 = seg_start[g], seg_start[g + 1]
        assert torch.equal(Y[r0:r1].cpu(), y[r0:r1])


@pytest.mark.parametrize("ydt", ["bf16", "f32"])
def test_lora_segmented_many_requests(ydt):
    """2300 requests (the pair table is written in 9 rounds of 256 requests),
    most of them 0-2 rows long, a few long ones, some without adapter: every
    pair's rows and adapter must come out of the table right."""
    rng = np.random.default_rng(2200)
    K, N, ranks = 272, 144, [8, 16, 64]
    lens = [int(rng.integers(0, 3)) if rng.random() < 0.97 else int(rng.integers(60, 200))
            for _ in range(2300)]
    M = int(sum(lens))
    seg_start = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    nseg = len(lens)
    seg_adapter = rng.integers(0, len(ranks), nseg).astype(np.int32)
    seg_adapter[rng.random(nseg) < 0.1] = -1
    x, xn = acts(rng, M, K, "bf16", factor=20.0)
    As = [cast_to(rng.normal(0, 0.01, (r, K)).astype(F32), "bf16") for r in ranks]
    Bs = [cast_to(rng.normal(0, 0.01, (N, r)).astype(F32), "bf16") for r in ranks]
    y = cast_to(rng.normal(0, 0.5, (M, N)).astype(F32), ydt)
    Ad = [t.cuda() for t in As]
    Bd = [t.cuda() for t in Bs]
    Y = y.cuda()
    ws = torch.empty(sq.sq_lora_workspace_bytes(M, K, 64), dtype=torch.uint8, device="cuda")
    sq.sq_lora_apply_segmented(x, dev(seg_start), dev(seg_adapter), sq.pointer_table(Ad, "cuda"),
                               sq.pointer_table(Bd, "cuda"), dev(np.array(ranks, np.int32)), 64, Y, ws)
    ref = O.lora_apply_segmented(y.float().numpy(), xn, "bf16", seg_start, seg_adapter,
                                 [t.float().numpy() for t in As], [t.float().numpy() for t in Bs],
                                 1.0, ydt)
    ok, rel = lora_close(Y.cpu().float().numpy(), ref)
    assert ok, rel
    none = np.zeros(M, bool)
    for g in np.nonzero(seg_adapter < 0)[0]:
        none[seg_start[g]:seg_start[g + 1]] = True
    assert torch.equal(Y.cpu()[torch.from_numpy(none)], y[torch.from_numpy(none)])


@pytest.mark.parametrize("case", ["no_adapter", "empty"])
def test_lora_segmented_no_pairs_leaves_y(case):
    """Requests that are all without an adapter, or all empty but one row
    span without adapter: the pair table holds no pair, every shrink block and
    expand tile exits, and Y is left as it was, bit for bit."""
    rng = np.random.default_rng(77)
    M, K, N, ranks = 200, 272, 144, [8, 16]
    if case == "no_adapter":
        seg_start = np.array([0, 10, 90, 200], np.int32)
        seg_adapter = np.array([-1, -1, -1], np.int32)
    else:
        seg_start = np.array([0, 0, 0, 200, 200], np.int32)
        seg_adapter = np.array([0, 1, -1, 1], np.int32)
    x, _ = acts(rng, M, K, "bf16", factor=20.0)
    As = [cast_to(rng.normal(0, 0.01, (r, K)).astype(F32), "bf16").cuda() for r in ranks]
    Bs = [cast_to(rng.normal(0, 0.01, (N, r)).astype(F32), "bf16").cuda() for r in ranks]
    y = cast_to(rng.normal(0, 0.5, (M, N)).astype(F32), "bf16")
    Y = y.cuda()
    ws = torch.empty(sq.sq_lora_workspace_bytes(M, K, 16), dtype=torch.uint8, device="cuda")
    sq.sq_lora_apply_segmented(x, dev(seg_start), dev(seg_adapter), sq.pointer_table(As, "cuda"),
                               sq.pointer_table(Bs, "cuda"), dev(np.array(ranks, np.int32)), 16, Y, ws)
    assert torch.equal(Y.cpu(), y)


def test_lora_segmented_single_adapter_equals_single():
    # both calls split K into the same 4 slices at this shape (300 rows, 4
    # requests), so one adapter over all rows gives the same result bit for bit
    rng = np.random.default_rng(9)
    M, K, N, r = 300, 1024, 256, 16
    x, xn, a, b, y = lora_inputs(rng, M, K, N, r, "bf16", "bf16")
    seg_start = np.array([0, 10, 11, 150, 300], np.int32)
    seg_adapter = np.zeros(4, np.int32)
    Y1 = y.cuda()
    Y2 = y.cuda()
    ws = torch.empty(sq.sq_lora_workspace_bytes(M, K, r), dtype=torch.uint8, device="cuda")
    sq.sq_lora_apply(x, a.cuda(), b.cuda(), Y1, ws)
    Ad, Bd = a.cuda(), b.cuda()
    sq.sq_lora_apply_segmented(x, dev(seg_start), dev(seg_adapter), sq.pointer_table([Ad], "cuda"),
                               sq.pointer_table([Bd], "cuda"), dev(np.array([r], np.int32)), r, Y2, ws)
    assert torch.equal(Y1, Y2)


# ---------------------------------------------------------------------------
# Determinism
# ---------------------------------------------------------------------------
def test_repeat_runs_are_bitwise_identical():
    rng = np.random.default_rng(21)
    M, K, N, r = 513, 4096, 1024, 16
    x, xn, a, b, y = lora_inputs(rng, M, K, N, r, "bf16", "bf16")
    w = cast_to(rng.normal(0, 0.02, (N, K)).astype(F32), "bf16").cuda()
    outs = []
    for _ in range(2):
        am = torch.zeros(K, dtype=torch.float32, device="cuda")
        s = torch.empty(K, dtype=torch.float32, device="cuda")
        Wq = torch.empty(N, K, dtype=torch.int8, device="cuda")
        wsc = torch.empty(N, dtype=torch.float32, device="cuda")
        Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
        asc = torch.empty(M, dtype=torch.float32, device="cuda")
        Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(sq.sq_lora_workspace_bytes(M, K, r), dtype=torch.uint8, device="cuda")
        sq.sq_calibrate_absmax(x, am)
        sq.sq_smooth_fold(am, w, 0.5, s, Wq, wsc)
        sq.sq_quant_per_token(x, s, Xq, asc)
        sq.sq_w8a8_gemm(Xq, Wq, asc, wsc, Y)
        sq.sq_lora_apply(x, a.cuda(), b.cuda(), Y, ws)
        outs.append([t.cpu() for t in (am, s, Wq, wsc, Xq, asc, Y)])
    for t1, t2 in zip(*outs):
        assert torch.equal(t1, t2)


# ---------------------------------------------------------------------------
# Fused path: stacked shrink, LoRA delta in the GEMM epilogue
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("r", [8, 24, 48, 128])
@pytest.mark.parametrize("xdt", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("M,K", [(1, 16), (33, 272), (300, 4096), (2048, 14336), (4096, 4368)])
def test_lora_shrink(r, xdt, M, K):
    """Covers one and two row tiles per wave, one and several k-chunks per
    slice, a K tail inside a chunk and a last rank tile that is partly empty."""
    rng = np.random.default_rng(r * 7 + M + K)
    x, xn = acts(rng, M, K, xdt, factor=20.0)
    a = cast_to(rng.normal(0, 0.01, (r, K)).astype(F32), "bf16")
    Tw = torch.zeros(M, r + 16, dtype=torch.bfloat16, device="cuda")
    T = Tw[:, :r]                                   # row stride wider than r
    ws = torch.empty(sq.sq_lora_workspace_bytes(M, K, r), dtype=torch.uint8, device="cuda")
    sq.sq_lora_shrink(x, a.cuda(), T, ws)
    an = a.float().numpy()
    ref = O.lora_shrink(xn, xdt, an).astype(np.float64)
    got = T.float().cpu().numpy().astype(np.float64)
    xb = xn if xdt == "bf16" else O.round_f32_to_bf16(xn)
    mag = np.abs(xb.astype(np.float64)) @ np.abs(an.astype(np.float64)).T
    # fp32 accumulation vs fp64, then one bf16 rounding on each side
    assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 2.0 ** -12 * mag)
    assert not Tw[:, r:].any()                      # nothing written past r


@pytest.mark.parametrize("out", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("mode", ["dynamic", "static"])
@pytest.mark.parametrize("M,N,K,r", [(33, 48, 272, 8), (300, 1024, 4096, 48), (64, 20480, 5120, 16),
                                     (257, 2048, 4096, 128), (40, 160, 80, 24)])
def test_gemm_lora(out, mode, M, N, K, r):
    rng = np.random.default_rng(M + N + K + r)
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    a = rng.uniform(1e-3, 5e-2, M if mode == "dynamic" else 1).astype(F32)
    w = rng.uniform(1e-5, 1e-3, N).astype(F32)
    t = cast_to(rng.normal(0, 0.5, (M, r)).astype(F32), "bf16")
    b = cast_to(rng.normal(0, 0.05, (N, r)).astype(F32), "bf16")
    Tw = torch.zeros(M, r + 8, dtype=torch.bfloat16)
    Tw[:, :r] = t
    Y = torch.zeros(M, N, dtype=DT[out], device="cuda")
    sq.sq_w8a8_gemm_lora(dev(xq), dev(wq), dev(a), dev(w), Tw.cuda()[:, :r], b.cuda(), Y, scale=0.5,
                         mode=mode)
    y = O.dequantize(O.int8_gemm(xq, wq), a if mode == "dynamic" else a[0], w, out)
    ref = O.lora_expand_add(y, t.float().numpy(), b.float().numpy(), 0.5, out)
    got = Y.cpu()
    got = got.float().numpy() if out != "f16" else got.numpy()
    ok, rel = lora_close(got, ref)
    assert ok, rel
    # T is given exactly, so the only difference is fp32 vs fp64 summation of r
    # products: 16-bit outputs are nearly all bit-identical; fp32 outputs (the
    # oracle adds in fp64 and rounds once) agree to a few fp32 ulps
    if out == "f32":
        g64, r64 = np.asarray(got, np.float64), np.asarray(ref, np.float64)
        assert np.all(np.abs(g64 - r64) <= 2.0 ** -20 * (np.abs(r64) + 0.5 * np.abs(
            t.float().numpy().astype(np.float64)) @ np.abs(b.float().numpy().astype(np.float64)).T))
    else:
        assert np.mean(np.asarray(got) != np.asarray(ref)) < 0.01


def test_gemm_lora_zero_b_equals_plain_gemm():
    rng = np.random.default_rng(77)
    M, N, K, r = 300, 2048, 4096, 32
    xq = dev(rng.integers(-127, 128, (M, K)).astype(np.int8))
    wq = dev(rng.integers(-127, 128, (N, K)).astype(np.int8))
    a = dev(rng.uniform(1e-3, 5e-2, M).astype(F32))
    w = dev(rng.uniform(1e-4, 1e-3, N).astype(F32))
    t = torch.randn(M, r, device="cuda").bfloat16()
    Y0 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    Y1 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    sq.sq_w8a8_gemm(xq, wq, a, w, Y0)
    sq.sq_w8a8_gemm_lora(xq, wq, a, w, t, torch.zeros(N, r, dtype=torch.bfloat16, device="cuda"), Y1)
    assert torch.equal(Y0, Y1)


def test_fused_group_matches_unfused():
    from synth.workloads import get_workload
    from w8a8_smoothquant_int8_amd.pipeline import LinearGroup
    wl = get_workload("llama3_8b_proj_m2048")
    inp = "attn_in"
    X = wl.x(inp).cuda()
    W = wl.w_group(inp).cuda()
    rows = wl.group_rows(inp)
    loras = {p: tuple(t.cuda() for t in wl.lora(p)) for p in rows}
    out = []
    for fuse in (True, False):
        g = LinearGroup(W, rows, wl.alpha, wl.out_dtype, wl.M, lora=loras, fuse=fuse)
        assert g.fused == fuse
        g.calibrate(wl.x_cal(inp).cuda())
        g.fold()
        out.append({p: t.clone() for p, t in g.forward(X).items()})
    for p in rows:
        ok, rel = lora_close(out[0][p].float().cpu().numpy(), out[1][p].float().cpu().numpy())
        assert ok, (p, rel)
        assert (out[0][p] != out[1][p]).float().mean().item() < 0.01


# ---------------------------------------------------------------------------
# The largest K the calls accept (32768): one row per block at 8 chunks per
# thread in the quantizer, the longest K loop in the GEMM.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_max_k_whole_path(dtype):
    K, M, N = 32768, 19, 48
    rng = np.random.default_rng(32768)
    x, xn = acts(rng, M, K, dtype, factor=30.0)
    w, wn = acts(rng, N, K, dtype, n_out=0, sigma=0.02)
    am = torch.zeros(K, dtype=torch.float32, device="cuda")
    sq.sq_calibrate_absmax(x, am)
    act_max = O.calibrate_absmax(xn)
    assert bits_equal(npf(am), act_max)
    s = torch.empty(K, dtype=torch.float32, device="cuda")
    Wq = torch.empty(N, K, dtype=torch.int8, device="cuda")
    ws = torch.empty(N, dtype=torch.float32, device="cuda")
    sq.sq_smooth_fold(am, w, 0.5, s, Wq, ws)
    s_ref = O.smoothing_scale(act_max, O.weight_absmax(wn), 0.5)
    assert bits_equal(npf(s), s_ref)
    wq_ref, ws_ref = O.fold_and_quantize_weights(wn, s_ref)
    assert bits_equal(Wq.cpu().numpy(), wq_ref) and bits_equal(npf(ws), ws_ref)
    Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    a = torch.empty(M, dtype=torch.float32, device="cuda")
    sq.sq_quant_per_token(x, s, Xq, a)
    xq_ref, a_ref = O.quantize_per_token(xn, s_ref)
    assert bits_equal(Xq.cpu().numpy(), xq_ref) and bits_equal(npf(a), a_ref)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    sq.sq_w8a8_gemm(Xq, Wq, a, ws, Y)
    y_ref = O.dequantize(O.int8_gemm(xq_ref, wq_ref), a_ref, ws_ref, "bf16")
    assert bits_equal(npf(Y), y_ref)


def test_max_k_extreme_accumulators():
    K = 32768                                         # |acc| up to K * 127^2 = 528,482,304 < 2^31
    xq = np.full((33, K), -127, np.int8)
    xq[::2] = 127
    wq = np.full((32, K), 127, np.int8)
    wq[1::4] = -127
    acc = torch.empty(33, 32, dtype=torch.int32, device="cuda")
    sq.sq_w8a8_gemm_i32(dev(xq), dev(wq), acc)
    ref = O.int8_gemm(xq, wq)
    assert np.abs(ref).max() == K * 127 * 127
    assert np.array_equal(acc.cpu().numpy(), ref)
