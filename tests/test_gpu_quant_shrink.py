"""Quant + LoRA shrink from one read of X (GPU) vs the oracle.

Bars: codes and per-token scales bit-exact (oracle and the path's quantizer);
T = bf16(fp32 sum of bf16(X) A^T) within one bf16 rounding plus the fp32
accumulation bound of the fp64 oracle value (the same bar as the separate
shrink), and nothing written past rank r in T.
"""
import numpy as np
import pytest
import torch

import oracle.sq_oracle as O
import w8a8_smoothquant_int8_amd as sq
from synth.workloads import cast_to

pytestmark = pytest.mark.gpu
F32 = np.float32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    assert sq.sq_query_support(0), "device 0 is not gfx950"


def run(rng, M, K, r, xdt, mode="dynamic", ld=None, zero_row=None):
    x = rng.standard_normal((M, K)).astype(F32)
    x[:, rng.choice(K, size=max(1, K // 300), replace=False)] *= 30.0
    if zero_row is not None:
        x[zero_row] = 0.0
    xt = cast_to(x, xdt)
    xn = xt.float().numpy()
    if ld is not None:
        wide = torch.zeros(M, ld, dtype=xt.dtype)
        wide[:, :K] = xt
        xd = wide.cuda()[:, :K]
    else:
        xd = xt.cuda()
    s = np.exp(np.random.default_rng(K).uniform(-1, 2, K)).astype(F32)
    a = cast_to(rng.normal(0, 0.01, (r, K)).astype(F32), "bf16")
    Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    if mode == "dynamic":
        asc = torch.empty(M, dtype=torch.float32, device="cuda")
        a_static = None
    else:
        a_static = O.static_activation_scale(O.calibrate_absmax(xn), s) * F32(0.8)   # some clipping
        asc = torch.tensor([a_static], dtype=torch.float32, device="cuda")
    Tw = torch.zeros(M, r + 16, dtype=torch.bfloat16, device="cuda")
    T = Tw[:, :r]
    sq.sq_quant_shrink(xd, torch.from_numpy(s).cuda(), Xq, asc, a.cuda(), T, mode=mode)
    torch.cuda.synchronize()
    if mode == "dynamic":
        rq, ra = O.quantize_per_token(xn, s)
        assert np.array_equal(asc.cpu().numpy().view(np.int32), ra.view(np.int32))
    else:
        rq, _ = O.quantize_per_tensor_static(xn, s, a_static)
    assert np.array_equal(Xq.cpu().numpy(), rq)
    an = a.float().numpy()
    ref = O.lora_shrink(xn, xdt, an).astype(np.float64)
    got = T.float().cpu().numpy().astype(np.float64)
    xb = xn if xdt == "bf16" else O.round_f32_to_bf16(xn)
    mag = np.abs(xb.astype(np.float64)) @ np.abs(an.astype(np.float64)).T
    assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 2.0 ** -12 * mag)
    assert not Tw[:, r:].any()
    return xd, s, Xq, asc, T


@pytest.mark.parametrize("xdt", ["bf16", "f16"])
@pytest.mark.parametrize("M,K,r", [(7, 272, 8), (33, 1024, 16), (100, 2048, 48), (2048, 4096, 48),
                                   (65, 4096, 128), (17, 4000, 32)])
def test_quant_shrink_matches_oracle(xdt, M, K, r):
    run(np.random.default_rng(M + K + r), M, K, r, xdt)


@pytest.mark.parametrize("M,K,r", [(130, 5120, 24), (48, 8192, 64), (17, 4112, 32), (256, 8192, 128)])
def test_quant_shrink_bf16_up_to_8192(M, K, r):
    run(np.random.default_rng(M + K + r), M, K, r, "bf16")


@pytest.mark.parametrize("M,K,r", [(40, 4096, 16), (23, 8192, 32)])
def test_quant_shrink_static(M, K, r):
    run(np.random.default_rng(M * K), M, K, r, "bf16", mode="static")


def test_quant_shrink_strided_and_zero_row():
    run(np.random.default_rng(2), 50, 2048, 32, "bf16", ld=2560, zero_row=7)


def test_quant_shrink_equals_quant_then_shrink_codes():
    """The codes and scales are the path quantizer's, bit for bit."""
    rng = np.random.default_rng(9)
    xd, s, Xq, asc, T = run(rng, 256, 4096, 48, "bf16")
    Xq2 = torch.empty_like(Xq)
    a2 = torch.empty_like(asc)
    sq.sq_quant_per_token(xd, torch.from_numpy(s).cuda(), Xq2, a2)
    assert torch.equal(Xq, Xq2) and torch.equal(asc, a2)
