"""Per-layer alpha sweep on the GPU vs the oracle's sweep.

Bars. The reference output sum (sum y_ref^2) is fp64 on both sides with
exact products: relative 1e-12. The error sums: the quantized outputs are
bit-exact with the oracle's when both sides hold the same smoothing vector,
which is guaranteed at alpha 0, 0.5 and 1 (a power of 1 or a square root,
correctly rounded): relative 1e-9 there. At other alphas the fp64 power on
the two sides may round a channel's s one fp32 ulp apart, which moves a few
codes by one: relative 1e-4. The chosen alpha must have the oracle's
smallest error (or one within 1e-4 of it).
"""
import numpy as np
import pytest
import torch

import oracle.sq_oracle as O
import w8a8_smoothquant_int8_amd as sq
from synth.workloads import cast_to, get_workload
from w8a8_smoothquant_int8_amd.pipeline import LinearGroup, alpha_sweep

pytestmark = pytest.mark.gpu
F32 = np.float32
ALPHAS = [0.0, 0.25, 0.4, 0.5, 0.6, 0.75, 0.85, 1.0]
EXACT = (0.0, 0.5, 1.0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    assert sq.sq_query_support(0), "device 0 is not gfx950"


def layer(rng, M, K, N, xt, wt, n_out=4, factor=40.0):
    x = rng.standard_normal((M, K)).astype(F32)
    x[:, rng.choice(K, size=min(n_out, K), replace=False)] *= factor
    w = (rng.standard_normal((N, K)) * 0.05).astype(F32)
    X, W = cast_to(x, xt), cast_to(w, wt)
    return X.cuda(), W.cuda(), X.float().numpy(), W.float().numpy()


def check_against_oracle(got, ref, alphas):
    assert got["ref"] == pytest.approx(ref["ref"], rel=1e-12)
    for i, a in enumerate(alphas):
        tol = 1e-9 if a in EXACT else 1e-4
        assert got["err"][i] == pytest.approx(ref["err"][i], rel=tol), a
    ib = alphas.index(got["best"])
    assert ref["rel"][ib] <= ref["rel"].min() * (1 + 1e-4)


@pytest.mark.parametrize("mode", ["dynamic", "static"])
@pytest.mark.parametrize("xt,wt", [("bf16", "bf16"), ("f16", "f16"), ("f32", "f32"), ("f32", "bf16")])
@pytest.mark.parametrize("M,K,N", [(37, 272, 48), (128, 1024, 256), (200, 4096, 320), (64, 2576, 160)])
def test_sweep_matches_oracle(M, K, N, xt, wt, mode):
    rng = np.random.default_rng(M + K + N)
    X, W, xn, wn = layer(rng, M, K, N, xt, wt)
    got = alpha_sweep(X, W, ALPHAS, mode=mode)
    ref = O.alpha_sweep(xn, wn, ALPHAS, mode=mode)
    check_against_oracle(got, ref, ALPHAS)


@pytest.mark.parametrize("mode", ["dynamic", "static"])
def test_sweep_exact_layer_zero_error_at_half(mode):
    # integer codes and power-of-two smoothing factors: alpha = 0.5 quantizes exactly
    rng = np.random.default_rng(5)
    M, K, N = 48, 64, 32
    cx = rng.integers(-100, 101, (M, K))
    cw = rng.integers(-100, 101, (N, K))
    cx[np.arange(M), rng.integers(0, K, M)] = 127
    cw[np.arange(N), rng.integers(0, K, N)] = -127
    c = np.maximum(np.abs(cx).max(0), np.abs(cw).max(0))
    cx[0, :] = np.where(np.abs(cx).max(0) < c, c, cx[0, :])
    cw[0, :] = np.where(np.abs(cw).max(0) < c, c, cw[0, :])
    sk = np.exp2(rng.integers(-3, 4, K)).astype(np.float64)
    x = torch.from_numpy((cx * sk).astype(F32)).to(torch.bfloat16).cuda()   # 8-bit codes: exact
    w = torch.from_numpy((cw / sk).astype(F32)).to(torch.bfloat16).cuda()
    got = alpha_sweep(x, w, [0.2, 0.5, 0.9], mode=mode)
    assert got["err"][1] == 0.0
    assert got["err"][0] > 0 and got["err"][2] > 0
    assert got["best"] == 0.5
    assert got["ref"] == float(np.sum((cx.astype(np.float64) @ cw.T.astype(np.float64)) ** 2))


def test_sweep_is_deterministic_and_leaves_inputs():
    rng = np.random.default_rng(9)
    X, W, _, _ = layer(rng, 256, 2048, 512, "bf16", "bf16")
    X0, W0 = X.clone(), W.clone()
    a = alpha_sweep(X, W, ALPHAS)
    b = alpha_sweep(X, W, ALPHAS)
    assert a == b
    assert torch.equal(X, X0) and torch.equal(W, W0)


def test_choose_alpha_sets_the_group_alpha():
    wl = get_workload("llama3_8b_proj_m2048")
    inp = "attn_in"
    W = wl.w_group(inp)
    g = LinearGroup(W.cuda(), wl.group_rows(inp), 0.5, wl.out_dtype, 64)
    xc = wl.x_cal(inp)[:128]
    r = g.choose_alpha(xc.cuda(), ALPHAS)
    assert g.alpha == r["best"]
    ref = O.alpha_sweep(xc.float().numpy(), W.float().numpy(), ALPHAS)
    check_against_oracle(r, ref, ALPHAS)


@pytest.mark.parametrize("name,inp", [("llama3_8b_proj_m2048", "attn_in"),
                                      ("opt13b_layer_prefill_m4096", "attn_in")])
def test_sweep_full_size_layer(name, inp):
    """A real layer group at full size: the whole calibration batch (512 rows)
    against the stacked Q/K/V weights, at three alphas."""
    wl = get_workload(name)
    xc, W = wl.x_cal(inp), wl.w_group(inp)
    alphas = [0.5, wl.alpha, 0.9] if wl.alpha != 0.5 else [0.3, 0.5, 0.9]
    got = alpha_sweep(xc.cuda(), W.cuda(), alphas)
    ref = O.alpha_sweep(xc.float().numpy(), W.float().numpy(), alphas)
    check_against_oracle(got, ref, alphas)
