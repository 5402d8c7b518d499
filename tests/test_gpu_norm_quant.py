"""Normalization with the folded 1/s fused with the quantizer (GPU) vs the oracle.

Bars. The folded weight and bias: bit-exact. Row statistics (mean, inverse
root): the GPU sums in fp64 in its own order, the oracle sums exactly, so
after the final rounding to fp32 they may differ by one ulp when the exact
value sits next to a rounding boundary; the test allows one ulp and at most
a few such rows. The codes and per-token scales are the integer decisions
taken from those statistics: bit-exact against the oracle run with the GPU's
statistics (and equal to the oracle's own wherever the statistics agree).
"""
import numpy as np
import pytest
import torch

import oracle.sq_oracle as O
import w8a8_smoothquant_int8_amd as sq
from synth.workloads import cast_to

pytestmark = pytest.mark.gpu
F32 = np.float32
EPS = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    assert sq.sq_query_support(0), "device 0 is not gfx950"


def residual(rng, M, K, dtype, mean_shift=0.0):
    h = (rng.standard_normal((M, K)) * 2.0 + mean_shift).astype(F32)
    h[:, rng.choice(K, size=max(1, K // 256), replace=False)] *= 40.0
    t = cast_to(h, dtype)
    return t.cuda(), t.float().numpy()


def norm_params(rng, K, dtype, kind):
    g = cast_to(rng.uniform(0.5, 1.5, K).astype(F32), dtype)
    b = cast_to((rng.standard_normal(K) * 0.2).astype(F32), dtype) if kind == "layer" else None
    s = np.exp(rng.uniform(-1.5, 2.0, K)).astype(F32)
    return g, b, s


def gpu_fold(g, b, s):
    K = g.numel()
    gd = g.cuda()
    bd = b.cuda() if b is not None else None
    go = torch.empty(K, dtype=torch.float32, device="cuda")
    bo = torch.empty(K, dtype=torch.float32, device="cuda") if b is not None else None
    sq.sq_fold_norm_weight(gd, bd, torch.from_numpy(s).cuda() if s is not None else None, go, bo)
    return go, bo


def ulps(a, b):
    a = np.ascontiguousarray(a, F32).view(np.int32).astype(np.int64)
    b = np.ascontiguousarray(b, F32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


def check(kind, hd, hn, go, bo, mode="dynamic", a_static=None):
    M, K = hn.shape
    Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    a = torch.empty(M, dtype=torch.float32, device="cuda")
    if mode == "static":
        a = torch.tensor([a_static], dtype=torch.float32, device="cuda")
    st = torch.empty(M, 2, dtype=torch.float32, device="cuda")
    sq.sq_norm_quant(hd, kind, go, bo, EPS, Xq, a, mode=mode, stats=st)
    gn, bn = go.cpu().numpy(), (bo.cpu().numpy() if bo is not None else None)
    mean_o, r_o = O.norm_stats(hn, kind, EPS)
    stn = st.cpu().numpy()
    mean_g, r_g = stn[:, 0].copy(), stn[:, 1].copy()
    um, ur = ulps(mean_g, mean_o), ulps(r_g, r_o)
    assert um.max() <= 1 and ur.max() <= 1
    assert np.count_nonzero(um) + np.count_nonzero(ur) <= max(2, M // 100)
    q_ref, a_ref, _ = O.norm_quant(hn, kind, gn, bn, EPS, mode=mode, a_static=a_static,
                                   stats=(mean_g, r_g))
    assert np.array_equal(Xq.cpu().numpy(), q_ref)
    if mode == "dynamic":
        assert np.array_equal(a.cpu().numpy().view(np.int32), a_ref.view(np.int32))
    return Xq, a, (mean_g, r_g)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_fold_norm_weight_bit_exact(dtype):
    rng = np.random.default_rng(1)
    K = 4112
    g, b, s = norm_params(rng, K, dtype, "layer")
    go, bo = gpu_fold(g, b, s)
    gr, br = O.fold_norm_weight(g.float().numpy(), b.float().numpy(), s)
    assert np.array_equal(go.cpu().numpy().view(np.int32), gr.view(np.int32))
    assert np.array_equal(bo.cpu().numpy().view(np.int32), br.view(np.int32))
    go1, _ = gpu_fold(g, None, None)                  # s = NULL: widened only
    assert np.array_equal(go1.cpu().numpy(), g.float().numpy())


SHAPES = [(7, 272), (33, 4096), (130, 5120), (65, 14336), (9, 16384), (48, 2576)]


@pytest.mark.parametrize("kind", ["rms", "layer"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M,K", SHAPES)
def test_norm_quant_matches_oracle(kind, dtype, M, K):
    rng = np.random.default_rng(M * 7 + K)
    hd, hn = residual(rng, M, K, dtype, mean_shift=0.5 if kind == "layer" else 0.0)
    g, b, s = norm_params(rng, K, dtype, kind)
    go, bo = gpu_fold(g, b, s)
    check(kind, hd, hn, go, bo)


@pytest.mark.parametrize("kind", ["rms", "layer"])
@pytest.mark.parametrize("M,K", [(5, 272), (40, 2048), (64, 4096)])
def test_norm_quant_fp32_input(kind, M, K):
    rng = np.random.default_rng(K + 3)
    hd, hn = residual(rng, M, K, "f32")
    g, b, s = norm_params(rng, K, "f32", kind)
    go, bo = gpu_fold(g, b, s)
    check(kind, hd, hn, go, bo)


@pytest.mark.parametrize("kind", ["rms", "layer"])
def test_norm_quant_static_scale_clips(kind):
    rng = np.random.default_rng(21)
    M, K = 96, 5120
    hd, hn = residual(rng, M, K, "f16")
    g, b, s = norm_params(rng, K, "f16", kind)
    go, bo = gpu_fold(g, b, s)
    Xq, _, _ = check(kind, hd, hn, go, bo, mode="static", a_static=F32(0.02))
    assert int(Xq.abs().max()) == 127


def test_norm_quant_strided_input_and_zero_rows():
    rng = np.random.default_rng(8)
    M, K, ld = 20, 1024, 1536
    h = torch.from_numpy(rng.standard_normal((M, ld)).astype(F32)).to(torch.bfloat16)
    h[3, :] = 0                                         # an all-zero row: r = 1/sqrt(eps), codes 0
    hd = h.cuda()[:, :K]
    hn = h[:, :K].float().numpy()
    g, _, s = norm_params(rng, K, "bf16", "rms")
    go, _ = gpu_fold(g, None, s)
    Xq, a, _ = check("rms", hd, hn, go, None)
    assert int(Xq[3].abs().max()) == 0 and float(a[3]) == 0.0


@pytest.mark.parametrize("kind", ["rms", "layer"])
def test_fused_equals_path_quantizer_for_power_of_two_s(kind):
    """With s a power of two, folding 1/s is exact, so the fused codes equal the
    path's own quantizer applied to the fp32 norm output (unfolded weight) and s."""
    rng = np.random.default_rng(13)
    M, K = 64, 4096
    hd, hn = residual(rng, M, K, "bf16")
    g, b, _ = norm_params(rng, K, "bf16", kind)
    s = np.exp2(rng.integers(-3, 4, K)).astype(F32)
    go, bo = gpu_fold(g, b, s)
    Xq, a, stats = check(kind, hd, hn, go, bo)
    x = O.norm_smooth(hn, kind, g.float().numpy(), None if b is None else b.float().numpy(), EPS,
                      stats)
    Xq2 = torch.empty_like(Xq)
    a2 = torch.empty_like(a)
    sq.sq_quant_per_token(torch.from_numpy(x).cuda(), torch.from_numpy(s).cuda(), Xq2, a2)
    assert torch.equal(Xq, Xq2) and torch.equal(a, a2)


@pytest.mark.parametrize("kind,dtype,M,K", [("rms", "bf16", 2048, 4096), ("layer", "f16", 4096, 5120),
                                            ("rms", "bf16", 8192, 8192)])
def test_norm_quant_full_size(kind, dtype, M, K):
    """The hidden-size inputs of the workloads (Llama-3-8B attention/MLP input,
    OPT-13B attention/FC1 input, Llama-2-70B MLP input), compared in full."""
    rng = np.random.default_rng(M + K)
    hd, hn = residual(rng, M, K, dtype)
    g, b, s = norm_params(rng, K, dtype, kind)
    go, bo = gpu_fold(g, b, s)
    check(kind, hd, hn, go, bo)


def test_pipeline_forward_norm_opt13b_attention():
    """The OPT-13B attention group (LayerNorm in front, fp16, no LoRA) at full
    size run straight from the residual stream: codes as the oracle's fused
    normalization gives them (with the GPU's row statistics), and the GEMM
    outputs on sampled rows and columns bit-exact."""
    from synth.workloads import get_workload, sample_rows
    from w8a8_smoothquant_int8_amd.pipeline import LinearGroup
    wl = get_workload("opt13b_layer_prefill_m4096")
    inp = "attn_in"
    rng = np.random.default_rng(3)
    K = wl.K_of(inp)
    hd, hn = residual(rng, wl.M, K, "f16", mean_shift=0.3)
    g, b, _ = norm_params(rng, K, "f16", "layer")
    W = wl.w_group(inp)
    rows = wl.group_rows(inp)
    grp = LinearGroup(W.cuda(), rows, wl.alpha, wl.out_dtype, wl.M)
    grp.calibrate(wl.x_cal(inp).cuda())
    grp.fold()
    grp.set_norm(g.cuda(), b.cuda(), "layer", EPS)
    grp.fold_norm()
    Y = {p: t.clone() for p, t in grp.forward_norm(hd).items()}
    torch.cuda.synchronize()
    s = grp.s.cpu().numpy()
    gf, bf = O.fold_norm_weight(g.float().numpy(), b.float().numpy(), s)
    st = torch.empty(wl.M, 2, dtype=torch.float32, device="cuda")
    Xq2 = torch.empty_like(grp.Xq)
    a2 = torch.empty_like(grp.a_scale)
    sq.sq_norm_quant(hd, "layer", grp.norm_g, grp.norm_b, EPS, Xq2, a2, stats=st)
    assert torch.equal(Xq2, grp.Xq)
    stn = st.cpu().numpy()
    q_ref, a_ref, _ = O.norm_quant(hn, "layer", gf, bf, EPS, stats=(stn[:, 0].copy(), stn[:, 1].copy()))
    assert np.array_equal(grp.Xq.cpu().numpy(), q_ref)
    m_rows = sample_rows(wl.M, 40)
    Wn = W.float().numpy()
    for p, (r0, r1) in rows.items():
        cols = sample_rows(r1 - r0, 48)
        wq, wsc = O.fold_and_quantize_weights(Wn[r0 + cols], s)
        y_ref = O.dequantize(O.int8_gemm(q_ref[m_rows], wq), a_ref[m_rows], wsc, wl.out_dtype)
        assert np.array_equal(Y[p].cpu().numpy()[np.ix_(m_rows, cols)], y_ref), p
