"""Static per-tensor quant with the clipped-code counter vs the oracle (GPU).

The codes must equal the oracle's bit for bit (and the plain static call's),
and the counter must equal the oracle's count of rounded codes beyond +-127,
exactly. Shapes cover every quantizer variant: one wave per row (K <= 4096
for 16-bit inputs), two and four waves per row (K <= 8192, 16384) and the
block kernel beyond, with ragged K (not a multiple of 512) and ragged M.
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


def batch(rng, M, K, dtype, sigma, cols, factor=60.0):
    x = (rng.standard_normal((M, K)) * sigma).astype(F32)
    x[:, cols] *= factor
    t = cast_to(x, dtype)
    return t.cuda(), t.float().numpy()


def static_setup(rng, K, dtype, cols, smooth=True):
    """Calibration batch -> act_max -> s -> the static scale, as the oracle computes them."""
    _, xcn = batch(rng, 64, K, dtype, 1.0, cols)
    s = np.exp(rng.uniform(-1, 2, K)).astype(F32) if smooth else None
    a = O.static_activation_scale(O.calibrate_absmax(xcn), s)
    return s, a


def run_clipped(x, s, a, counter):
    M, K = x.shape
    Xq = torch.empty(M, K, dtype=torch.int8, device="cuda")
    sd = torch.from_numpy(s).cuda() if s is not None else None
    ad = torch.tensor([a], dtype=torch.float32, device="cuda")
    sq.sq_quant_static_clipped(x, sd, ad, Xq, counter)
    return Xq


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("M,K", [(7, 272), (33, 4096), (300, 5120), (65, 14336), (17, 20480),
                                 (129, 2576)])
def test_clip_count_and_codes_match_oracle(dtype, M, K):
    rng = np.random.default_rng(100 + K + M)
    cols = rng.choice(K, size=max(1, K // 200), replace=False)
    s, a = static_setup(rng, K, dtype, cols)
    # a batch three times wider than the calibration batch: many codes clip
    x, xn = batch(rng, M, K, dtype, 3.0, cols)
    counter = torch.zeros(1, dtype=torch.int64, device="cuda")
    Xq = run_clipped(x, s, a, counter)
    rq, clipped = O.quantize_per_tensor_static(xn, s, a)
    assert clipped > 0
    assert np.array_equal(Xq.cpu().numpy(), rq)
    assert int(counter.item()) == clipped
    # the plain static call gives the same codes
    Xq2 = torch.empty_like(Xq)
    sq.sq_quant_per_token(x, torch.from_numpy(s).cuda(), Xq2,
                          torch.tensor([a], dtype=torch.float32, device="cuda"), mode="static")
    assert torch.equal(Xq, Xq2)


@pytest.mark.parametrize("K", [4096, 14336])
def test_clip_count_zero_on_calibration_batch(K):
    # the scale comes from this very batch, so |x_s / a| <= 127 and nothing clips
    rng = np.random.default_rng(7 + K)
    cols = rng.choice(K, size=K // 200, replace=False)
    x, xn = batch(rng, 96, K, "bf16", 1.0, cols)
    s = np.exp(rng.uniform(-1, 2, K)).astype(F32)
    a = O.static_activation_scale(O.calibrate_absmax(xn), s)
    counter = torch.zeros(1, dtype=torch.int64, device="cuda")
    Xq = run_clipped(x, s, a, counter)
    rq, clipped = O.quantize_per_tensor_static(xn, s, a)
    assert clipped == 0
    assert int(counter.item()) == 0
    assert np.array_equal(Xq.cpu().numpy(), rq)
    assert int(Xq.abs().max()) == 127


def test_clip_counter_accumulates_over_calls():
    K = 5120
    rng = np.random.default_rng(11)
    cols = rng.choice(K, size=20, replace=False)
    s, a = static_setup(rng, K, "f16", cols)
    counter = torch.zeros(1, dtype=torch.int64, device="cuda")
    total = 0
    for M, sigma in ((40, 2.0), (9, 4.0), (128, 1.5)):
        x, xn = batch(rng, M, K, "f16", sigma, cols)
        Xq = run_clipped(x, s, a, counter)
        rq, clipped = O.quantize_per_tensor_static(xn, s, a)
        assert np.array_equal(Xq.cpu().numpy(), rq)
        total += clipped
    assert total > 0
    assert int(counter.item()) == total


def test_clip_ties_and_no_smoothing():
    # s = NULL, a = 1: codes are rne(x); 127.5 and -127.5 round to +-128 (even) and clip,
    # 126.5 rounds to 126 and does not; 127.49 stays 127.
    K = 16
    row = np.array([126.4, 127.4, 127.5, 128.6, -127.5, -127.49, 200.0, -1000.0,
                    126.5, 0.0, 1.0, -1.0, 127.0, -127.0, 128.5, 3.0], F32)
    x = torch.from_numpy(np.stack([row, -row])).cuda()
    counter = torch.zeros(1, dtype=torch.int64, device="cuda")
    Xq = run_clipped(x, None, F32(1.0), counter)
    rq, clipped = O.quantize_per_tensor_static(np.stack([row, -row]), None, F32(1.0))
    assert clipped == 12
    assert int(counter.item()) == 12
    assert np.array_equal(Xq.cpu().numpy(), rq)


def test_zero_scale_clips_nothing():
    K = 4096
    rng = np.random.default_rng(3)
    x, _ = batch(rng, 8, K, "bf16", 1.0, [0])
    counter = torch.zeros(1, dtype=torch.int64, device="cuda")
    Xq = run_clipped(x, None, F32(0.0), counter)
    assert int(Xq.abs().max()) == 0
    assert int(counter.item()) == 0


def test_empty_batch_leaves_counter():
    # M = 0 through the C ABI with real buffers (torch gives empty tensors a null pointer)
    import ctypes
    counter = torch.full((1,), 5, dtype=torch.int64, device="cuda")
    x = torch.ones(4, 256, dtype=torch.bfloat16, device="cuda")
    Xq = torch.full((4, 256), 7, dtype=torch.int8, device="cuda")
    a = torch.ones(1, dtype=torch.float32, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = sq.lib().sq_quant_static_clipped(P(x), sq.SQ_BF16, 0, 256, 256, None, P(a), P(Xq),
                                          P(counter), None)
    assert rc == sq.SQ_OK
    torch.cuda.synchronize()
    assert int(counter.item()) == 5
    assert int(Xq.min()) == 7 and int(Xq.max()) == 7


@pytest.mark.parametrize("inp", ["attn_in", "fc2_in"])
def test_range_check_on_opt13b_prefill(inp):
    """Full-size OPT-13B layer input (M = 4096), static mode through the pipeline:
    the clip count over the whole batch equals the oracle's; a batch whose values
    are far beyond the calibrated range fails the range check and falls back to
    per-token dynamic scales, giving exactly the dynamic forward pass."""
    from synth.workloads import get_workload
    from w8a8_smoothquant_int8_amd.pipeline import LinearGroup
    wl = get_workload("opt13b_layer_prefill_m4096")
    X, Xc, W = wl.x(inp), wl.x_cal(inp), wl.w_group(inp)
    rows = wl.group_rows(inp)
    g = LinearGroup(W.cuda(), rows, wl.alpha, wl.out_dtype, wl.M, modes=("dynamic", "static"))
    g.calibrate(Xc.cuda())
    g.fold()
    Xd = X.cuda()
    Y, rate, fell_back = g.forward_static_checked(Xd, max_rate=1.0)
    assert not fell_back
    s, a = g.s.cpu().numpy(), g.static_scale.cpu().numpy()[0]
    xq, clipped = O.quantize_per_tensor_static(X.float().numpy(), s, a)
    assert np.array_equal(g.Xq.cpu().numpy(), xq)
    assert rate == clipped / X.numel()
    assert g.clip_rate() == rate

    # a spike: the batch scaled by 8 clips far more than the check allows
    g.reset_clips()
    spike = (Xd.float() * 8).to(Xd.dtype)
    Y, rate, fell_back = g.forward_static_checked(spike)
    assert fell_back and rate > 1e-3
    got = {p: t.clone() for p, t in Y.items()}
    ref = g.forward(spike, "dynamic")
    for p in rows:
        assert torch.equal(got[p], ref[p]), p
