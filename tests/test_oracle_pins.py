"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test ties one oracle function to something the oracle does not compute
itself: the values the SmoothQuant explainer prints for its worked example, a
hand-worked 4x4 example whose every step is exact in binary, closed forms of
the scale formula, invariants the method guarantees, library routines for
special cases, and a pure-Python brute force (tests/brute.py) on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.sq_oracle as O
import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# 1. The page's own worked example (SmoothQuant explainer, "A worked example").
# ---------------------------------------------------------------------------
def test_page_worked_example_unsmoothed():
    g = _golden("smoothquant_worked_example.json")
    x = np.array([g["layer"]["x"]], F32)
    w = np.array([g["layer"]["w"]], F32)
    # exact output of the layer
    assert float((x.astype(np.float64) @ w.astype(np.float64).T)[0, 0]) == g["layer"]["exact_output"]
    q, a = O.quantize_per_token(x, None)
    u = g["unsmoothed"]
    assert abs(float(a[0]) - u["scale_approx"]) <= u["scale_abs_tol"]
    assert abs(float(x[0, 1] / a[0]) - u["quotient_approx"]) <= u["quotient_abs_tol"]
    assert int(q[0, 1]) == u["code_small_channel"]
    assert abs(float(q[0, 1]) * float(a[0]) - u["dequant_approx"]) <= u["dequant_abs_tol"]
    # a larger outlier wipes out the small channel
    o = g["outlier_400"]
    q4, a4 = O.quantize_per_token(np.array([o["x"]], F32), None)
    assert abs(float(a4[0]) - o["scale_approx"]) <= o["scale_abs_tol"]
    assert int(q4[0, 1]) == o["code_small_channel"]


def test_page_worked_example_smoothed():
    g = _golden("smoothquant_worked_example.json")
    sm = g["smoothed"]
    x = np.array([g["layer"]["x"]], F32)
    w = np.array([g["layer"]["w"]], F32)
    s = np.array(sm["s"], F32)
    xs = O.smooth_activations(x, s)
    assert xs[0].tolist() == sm["x_smoothed"]
    assert (w * s[None, :])[0].tolist() == sm["w_scaled"]
    assert float((xs.astype(np.float64) @ (w * s).astype(np.float64).T)[0, 0]) == sm["output"]
    q, a = O.quantize_per_token(x, s)
    assert abs(float(a[0]) - sm["scale_approx"]) <= sm["scale_abs_tol"]
    assert int(q[0, 1]) == sm["code_small_channel"]
    assert int(q[0, 0]) == 127


# ---------------------------------------------------------------------------
# 2. Hand-worked 4x4 example, alpha = 0.5, every value dyadic.
#    act_max = [256, 4, 16, 1] and w_max = [1/4, 1, 1/4, 1], so
#    s = sqrt(a)/sqrt(w) = [16/(1/2), 2/1, 4/(1/2), 1/1] = [32, 2, 8, 1].
#    Row 0 of X/s = [7.9375, 0.15625, -0.21875, 0.03125]; its absmax / 127 is
#    exactly 1/16, and the quotients 2.5, -3.5, 0.5 are exact ties, which
#    half-to-even rounds to 2, -4, 0 (half-away would give 3, -4, 1).
#    Weight row 1 of W*s = [-4, 1, -2, 1] has scale 4/127; -2 / (4/127) rounds
#    in fp32 to exactly -63.5, a tie that goes to -64.
# ---------------------------------------------------------------------------
X44 = [[254, 0.3125, -1.75, 0.03125], [-256, 4, 3, -0.5], [64, -1, 16, 1], [-32, 0.5, -1, 0.75]]
W44 = [[0.25, 1, 0.125, -0.5], [-0.125, 0.5, -0.25, 1], [0.0625, -1, 0.25, 0.25],
       [-0.25, 0.25, 0.0625, -1]]


def test_hand_4x4_example():
    x = np.array(X44, F32)
    w = np.array(W44, F32)
    r = O.smoothquant_linear(x, "f32", w, x, 0.5, "bf16")
    assert r["act_max"].tolist() == [256, 4, 16, 1]
    assert r["w_max"].tolist() == [0.25, 1, 0.25, 1]
    assert r["s"].tolist() == [32, 2, 8, 1]
    assert float(r["a_scale"][0]) == 0.0625
    assert r["a_scale"].tolist() == [F32(v) / F32(127) for v in (7.9375, 8, 2, 1)]
    assert r["w_scale"].tolist() == [F32(v) / F32(127) for v in (8, 4, 2, 8)]
    assert r["xq"].tolist() == [[127, 2, -4, 0], [-127, 32, 6, -8], [127, -32, 127, 64],
                                [-127, 32, -16, 95]]
    assert r["wq"].tolist() == [[127, 32, 16, -8], [-127, 32, -64, 32], [127, -127, 127, 16],
                                [-127, 8, 8, -16]]
    # acc = Xq Wq^T, worked by hand: e.g. acc[0,0] = 127*127 + 2*32 - 4*16 + 0 = 16129
    assert r["acc"].tolist() == [[16129, -15809, 15367, -16145], [-14945, 16513, -19559, 16561],
                                 [16625, -23233, 37346, -16393], [-16121, 21217, -20705, 14737]]
    # acc[0,0] * (1/16) * (8/127) = 16129 / 254 = 63.5 exactly
    assert float(r["y"][0, 0]) == 63.5
    assert r["y"].tolist() == [[63.5, -31.125, 15.125, -63.5], [-59.25, 32.75, -19.375, 65.5],
                               [16.5, -11.5, 9.25, -16.25], [-8, 5.25, -2.5625, 7.3125]]


def test_hand_4x4_smoothing_is_exact_with_power_of_two_scales():
    # With s a power of two, X/s and W*s are exact, so the smoothed product equals X W^T exactly.
    x = np.array(X44, np.float64)
    w = np.array(W44, np.float64)
    s = np.array([32, 2, 8, 1], np.float64)
    assert np.array_equal((x / s) @ (w * s).T, x @ w.T)


# ---------------------------------------------------------------------------
# 3. Division, not reciprocal-multiply (one row, s = 1).
#    [2.25, 1.125]: scale = fp32(2.25/127); fp32(1.125/scale) = 63.499996 -> 63,
#    while 1.125 * fp32(127/2.25) = 63.5 -> 64.
#    [3.75, 1.875]: fp32(1.875/fp32(3.75/127)) = 63.5 exactly -> 64 (even),
#    while the reciprocal form gives 63.499996 -> 63.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("row,codes", [([2.25, 1.125], [127, 63]), ([3.75, 1.875], [127, 64])])
def test_division_vectors(row, codes):
    q, a = O.quantize_per_token(np.array([row], F32), None)
    assert q[0].tolist() == codes
    recip = np.rint(F32(row[1]) * (F32(127) / F32(row[0])))
    assert int(recip) != codes[1]   # the vector really separates the two forms


# ---------------------------------------------------------------------------
# 4. Brute force on tiny random inputs: every intermediate, bit for bit.
# ---------------------------------------------------------------------------
def _tiny_case(seed, M, K, N, dtype):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(F32)
    xc = rng.standard_normal((max(M, 3), K)).astype(F32)
    out_col = rng.integers(0, K)
    x[:, out_col] *= 40
    xc[:, out_col] *= 40
    w = rng.normal(0, 0.02, (N, K)).astype(F32)
    if dtype == "bf16":
        x, xc, w = (torch.from_numpy(t).bfloat16().float().numpy() for t in (x, xc, w))
    elif dtype == "f16":
        x, xc, w = (t.astype(np.float16).astype(F32) for t in (x, xc, w))
    return x, xc, w


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("alpha", [0.5, 0.8, 0.25, 1.0, 0.0])
def test_brute_force_pipeline(seed, alpha):
    rng = np.random.default_rng(1000 + seed)
    M, K, N = (int(v) for v in rng.integers(1, 9, size=3))
    dtype = ["f32", "bf16", "f16"][seed % 3]
    out = ["bf16", "f16", "f32"][(seed // 3) % 3]
    mode = "static" if seed % 2 else "dynamic"
    x, xc, w = _tiny_case(seed, M, K, N, dtype)
    r = O.smoothquant_linear(x, dtype, w, xc, alpha, out, mode=mode)
    b = brute.pipeline(x.tolist(), w.tolist(), xc.tolist(), alpha, mode=mode, out=out)
    assert r["act_max"].tolist() == b["act_max"]
    assert r["w_max"].tolist() == b["w_max"]
    assert r["s"].tolist() == b["s"]
    assert r["w_scale"].tolist() == b["w_scale"]
    assert r["wq"].tolist() == b["wq"]
    a = r["a_scale"]
    assert (np.full(M, a) if np.ndim(a) == 0 else a).tolist() == b["a_scale"]
    assert r["xq"].tolist() == b["xq"]
    assert r["acc"].tolist() == b["acc"]
    assert r["y"].astype(np.float64).tolist() == b["y"]


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_lora(seed):
    rng = np.random.default_rng(50 + seed)
    M, K, N, R = (int(v) for v in rng.integers(1, 7, size=4))
    in_dtype = "bf16" if seed % 2 else "f32"
    x = rng.standard_normal((M, K)).astype(F32)
    if in_dtype == "bf16":
        x = O.round_f32_to_bf16(x)
    a = O.round_f32_to_bf16(rng.normal(0, 0.3, (R, K)).astype(F32))
    bm = O.round_f32_to_bf16(rng.normal(0, 0.3, (N, R)).astype(F32))
    y = O.round_f32_to_bf16(rng.standard_normal((M, N)).astype(F32))
    scale = [1.0, 0.5, 2.0][seed % 3]
    t = O.lora_shrink(x, in_dtype, a)
    yl = O.lora_expand_add(y, t, bm, scale, "bf16")
    tb, yb = brute.lora(y.tolist(), x.tolist(), a.tolist(), bm.tolist(), scale,
                        x_is_bf16=(in_dtype == "bf16"))
    assert t.tolist() == tb
    assert yl.tolist() == yb


# ---------------------------------------------------------------------------
# 5. Closed forms and invariants of the scale formula (SmoothQuant, Step 3).
# ---------------------------------------------------------------------------
def _rand_maxima(seed, K=4096):
    rng = np.random.default_rng(seed)
    a = np.exp(rng.uniform(np.log(0.5), np.log(400), K)).astype(F32)
    w = np.exp(rng.uniform(np.log(1e-3), np.log(0.2), K)).astype(F32)
    return a, w


def test_scale_alpha_one_and_zero():
    a, w = _rand_maxima(1)
    assert np.array_equal(O.smoothing_scale(a, w, 1.0), a)               # a^1 / w^0
    assert np.array_equal(O.smoothing_scale(a, w, 0.0),                  # a^0 / w^1
                          (1.0 / w.astype(np.float64)).astype(F32))


def test_scale_clamps():
    # zero channels: both maxima clamp to 1e-5, so s = 1e-5^a / 1e-5^(1-a)
    s = O.smoothing_scale(np.array([0.0], F32), np.array([0.0], F32), 0.8)
    assert s[0] == F32(1e-5 ** 0.8 / 1e-5 ** 0.2)
    # s itself is clamped below at 1e-5
    s = O.smoothing_scale(np.array([1e-5], F32), np.array([100.0], F32), 1.0)
    assert s[0] == F32(1e-5)


@pytest.mark.parametrize("alpha", [0.8, 0.3, 0.65])
def test_scale_matches_exact_decimal(alpha):
    a, w = _rand_maxima(2, K=400)
    s = O.smoothing_scale(a, w, alpha)
    exact = [brute.scale_s_decimal(float(ai), float(wi), alpha) for ai, wi in zip(a, w)]
    assert s.tolist() == exact


def test_scale_alpha_half_balances_channel_maxima():
    # At alpha = 0.5, max|X_s[:, j]| = a_j / s_j and max|W_s[:, j]| = w_j * s_j
    # both equal sqrt(a_j * w_j) up to rounding ("balanced", Step 3).
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 512)).astype(F32)
    x[:, :8] *= 80
    w = rng.normal(0, 0.02, (128, 512)).astype(F32)
    am, wm = O.calibrate_absmax(x), O.weight_absmax(w)
    s = O.smoothing_scale(am, wm, 0.5)
    xs_max = np.abs(O.smooth_activations(x, s)).max(axis=0).astype(np.float64)
    ws_max = np.abs(w * s).max(axis=0).astype(np.float64)
    geo = np.sqrt(am.astype(np.float64) * wm.astype(np.float64))
    assert np.allclose(xs_max, geo, rtol=3e-7, atol=0)
    assert np.allclose(ws_max, geo, rtol=3e-7, atol=0)
    # and the smoothed activation profile is flatter than before (diagnostics section)
    assert xs_max.max() / xs_max.min() < am.max() / am.min()


def test_smoothing_equivalence_fp64():
    # Step 2: (X diag(s)^-1)(diag(s) W^T) == X W^T in exact arithmetic.
    rng = np.random.default_rng(4)
    x = rng.standard_normal((32, 256))
    x[:, 3] *= 60
    w = rng.normal(0, 0.02, (48, 256))
    s = O.smoothing_scale(O.calibrate_absmax(x.astype(F32)), O.weight_absmax(w.astype(F32)), 0.5)
    s = s.astype(np.float64)
    lhs = (x / s) @ (w * s).T
    ref = x @ w.T
    assert np.linalg.norm(lhs - ref) / np.linalg.norm(ref) < 1e-12


# ---------------------------------------------------------------------------
# 6. Quantizer invariants (Step 6).
# ---------------------------------------------------------------------------
def test_quantizer_invariants():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((200, 333)).astype(F32)
    x[:, 7] *= 90
    x[5] = 0.0                        # a zero row: scale 0, codes 0
    s = np.exp(rng.uniform(-2, 2, 333)).astype(F32)
    q, a = O.quantize_per_token(x, s)
    xs = O.smooth_activations(x, s)
    assert a[5] == 0 and not q[5].any()
    nz = np.abs(x).max(axis=1) > 0
    assert np.all(np.abs(q[nz]).max(axis=1) == 127)          # every nonzero row reaches 127
    assert np.abs(q.astype(np.int32)).max() <= 127
    err = np.abs(xs.astype(np.float64) - q.astype(np.float64) * a[:, None].astype(np.float64))
    assert np.all(err <= a[:, None].astype(np.float64) * (0.5 + 1e-6))


def test_static_scale_no_clip_on_own_batch_and_clips_beyond():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((100, 64)).astype(F32)
    s = np.exp(rng.uniform(-1, 1, 64)).astype(F32)
    a = O.static_activation_scale(O.calibrate_absmax(x), s)
    q, clipped = O.quantize_per_tensor_static(x, s, a)
    assert clipped == 0 and np.abs(q).max() == 127
    # the static scale equals the per-tensor absmax of the smoothed batch / 127
    assert a == F32(np.abs(O.smooth_activations(x, s)).max() / F32(127))
    x2 = x.copy()
    x2[0, 0] = 10 * np.abs(x).max()
    q2, clipped2 = O.quantize_per_tensor_static(x2, s, a)
    assert clipped2 >= 1 and q2[0, 0] in (127, -127)


def test_calibration_running_max_is_order_independent():
    rng = np.random.default_rng(7)
    batches = [rng.standard_normal((int(n), 96)).astype(F32) for n in rng.integers(1, 40, 5)]
    run = None
    for b in batches:
        run = O.calibrate_absmax(b, run)
    run_rev = None
    for b in batches[::-1]:
        run_rev = O.calibrate_absmax(b[::-1], run_rev)
    assert np.array_equal(run, run_rev)
    assert np.array_equal(run, np.abs(np.concatenate(batches)).max(axis=0))


# ---------------------------------------------------------------------------
# 7. INT8 GEMM exactness (Step 7).
# ---------------------------------------------------------------------------
def test_int8_gemm_matches_integer_matmul():
    rng = np.random.default_rng(8)
    xq = rng.integers(-127, 128, (37, 1024)).astype(np.int8)
    wq = rng.integers(-127, 128, (29, 1024)).astype(np.int8)
    ref = xq.astype(np.int64) @ wq.astype(np.int64).T   # numpy's integer matmul (no float)
    assert np.array_equal(O.int8_gemm(xq, wq), ref)


def test_int8_gemm_extreme_magnitude():
    K = 28672          # largest K of the workloads: |acc| <= K * 127^2 < 2^31
    xq = np.full((2, K), 127, np.int8)
    xq[1] = -127
    wq = np.full((3, K), 127, np.int8)
    wq[2, ::2] = -127
    acc = O.int8_gemm(xq, wq)
    assert acc[0, 0] == K * 127 * 127 and acc[1, 1] == -K * 127 * 127
    assert acc[0, 2] == 0


def test_dequant_bf16_and_f16_rounding():
    rng = np.random.default_rng(9)
    acc = rng.integers(-2 ** 27, 2 ** 27, (5, 7)).astype(np.int32)   # > 2^24: int->fp32 rounds
    a = rng.uniform(1e-5, 1e-3, 5).astype(F32)
    w = rng.uniform(1e-5, 1e-3, 7).astype(F32)
    for out in ("bf16", "f16", "f32"):
        y = O.dequantize(acc, a, w, out)
        rnd = {"bf16": brute.bf16, "f16": brute.f16, "f32": lambda v: v}[out]
        exp = [[rnd(brute.f32(brute.f32(brute.f32(float(acc[m, n])) * float(a[m])) * float(w[n])))
                for n in range(7)] for m in range(5)]
        assert y.astype(np.float64).tolist() == exp


# ---------------------------------------------------------------------------
# 8. Rounding helpers against independent definitions.
# ---------------------------------------------------------------------------
def test_round_f32_to_bf16_matches_torch_cast():
    rng = np.random.default_rng(10)
    v = rng.standard_normal(200000).astype(F32) * np.exp(rng.uniform(-20, 20, 200000)).astype(F32)
    # plant exact ties: low 16 bits == 0x8000
    bits = v.view(np.uint32).copy()
    bits[:5000] = (bits[:5000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    v = bits.view(F32)
    ref = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
    assert np.array_equal(O.round_f32_to_bf16(v), ref)


def test_round_f64_to_bf16_single_rounding():
    rng = np.random.default_rng(11)
    v = rng.standard_normal(3000) * np.exp(rng.uniform(-10, 10, 3000))
    got = O.round_f64_to_bf16(v)
    assert [float(g) for g in got] == [brute.bf16(float(x)) for x in v]
    # a value just above a bf16 tie in fp64 that rounds to the tie in fp32 (double rounding)
    x = 1.0 + 2 ** -8 + 2 ** -30
    assert float(O.round_f64_to_bf16(np.array([x]))[0]) == 1.0 + 2 ** -7


# ---------------------------------------------------------------------------
# 9. LoRA special cases (Pitch of the LoRA-for-SmoothQuant issue).
# ---------------------------------------------------------------------------
def _lora_case(seed=12, M=40, K=64, N=24, r=8):
    rng = np.random.default_rng(seed)
    x = O.round_f32_to_bf16(rng.standard_normal((M, K)).astype(F32))
    a = O.round_f32_to_bf16(rng.normal(0, 0.01, (r, K)).astype(F32))
    b = O.round_f32_to_bf16(rng.normal(0, 0.01, (N, r)).astype(F32))
    y = O.round_f32_to_bf16(rng.standard_normal((M, N)).astype(F32))
    return x, a, b, y


def test_lora_zero_b_leaves_output_unchanged():
    x, a, b, y = _lora_case()
    assert np.array_equal(O.lora_apply(y, x, "bf16", a, np.zeros_like(b), 1.0, "bf16"), y)


def test_lora_matches_fp64_textbook_within_bf16():
    x, a, b, y = _lora_case()
    got = O.lora_apply(y, x, "bf16", a, b, 1.0, "bf16")
    t = x.astype(np.float64) @ a.T.astype(np.float64)
    exact = y.astype(np.float64) + t @ b.T.astype(np.float64)
    # bound: one bf16 rounding of the result plus one bf16 rounding of each T entry
    bound = 2.0 ** -8 * np.abs(exact) + 2.0 ** -8 * (np.abs(t) @ np.abs(b.T.astype(np.float64)))
    assert np.all(np.abs(got - exact) <= bound)


def test_segmented_reduces_to_single_adapter():
    x, a, b, y = _lora_case(M=100)
    a2 = O.round_f32_to_bf16(np.random.default_rng(1).normal(0, 0.01, (16, 64)).astype(F32))
    b2 = O.round_f32_to_bf16(np.random.default_rng(2).normal(0, 0.01, (24, 16)).astype(F32))
    seg = [0, 30, 31, 77, 100]
    # all segments on one adapter == single-adapter LoRA
    one = O.lora_apply_segmented(y, x, "bf16", seg, [0, 0, 0, 0], [a, a2], [b, b2], 1.0, "bf16")
    assert np.array_equal(one, O.lora_apply(y, x, "bf16", a, b, 1.0, "bf16"))
    # mixed: each segment equals single-adapter LoRA on its rows; adapter -1 leaves rows alone
    mix = O.lora_apply_segmented(y, x, "bf16", seg, [1, -1, 0, 1], [a, a2], [b, b2], 1.0, "bf16")
    assert np.array_equal(mix[:30], O.lora_apply(y[:30], x[:30], "bf16", a2, b2, 1.0, "bf16"))
    assert np.array_equal(mix[30:31], y[30:31])
    assert np.array_equal(mix[31:77], O.lora_apply(y[31:77], x[31:77], "bf16", a, b, 1.0, "bf16"))
    assert np.array_equal(mix[77:], O.lora_apply(y[77:], x[77:], "bf16", a2, b2, 1.0, "bf16"))


# ---------------------------------------------------------------------------
# 10. Planted mistakes: each plausible slip in the oracle must fail a pin.
# ---------------------------------------------------------------------------
def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_planted_mistakes_are_caught(monkeypatch):
    orig_qr = O.quantize_rows

    def half_away(t, scale):
        t = np.asarray(t, F32)
        sc = np.asarray(scale, F32).reshape(-1, 1)
        v = t / sc
        return np.clip(np.sign(v) * np.floor(np.abs(v) + 0.5), -127, 127).astype(np.int8)
    monkeypatch.setattr(O, "quantize_rows", half_away)
    assert _fails(test_hand_4x4_example)
    monkeypatch.setattr(O, "quantize_rows", orig_qr)

    def recip(t, scale):
        t = np.asarray(t, F32)
        sc = np.asarray(scale, F32).reshape(-1, 1)
        inv = np.where(sc != 0, F32(1) / np.where(sc != 0, sc, 1), 0).astype(F32)
        return np.clip(np.rint(t * inv), -127, 127).astype(np.int8)
    monkeypatch.setattr(O, "quantize_rows", recip)
    assert _fails(lambda: test_division_vectors([2.25, 1.125], [127, 63]))
    monkeypatch.setattr(O, "quantize_rows", orig_qr)

    orig_ss = O.smoothing_scale
    monkeypatch.setattr(O, "smoothing_scale",
                        lambda a, w, al: orig_ss(a, w, 1.0 - al))     # alpha swapped
    assert _fails(lambda: test_brute_force_pipeline(0, 0.8))
    monkeypatch.setattr(O, "smoothing_scale", orig_ss)

    orig_sa = O.smooth_activations
    monkeypatch.setattr(O, "smooth_activations",
                        lambda x, s: np.asarray(x, F32) * np.asarray(s, F32)[None, :])  # wrong side
    assert _fails(test_hand_4x4_example)
    monkeypatch.setattr(O, "smooth_activations", orig_sa)

    orig_gemm = O.int8_gemm
    monkeypatch.setattr(O, "int8_gemm", lambda xq, wq: orig_gemm(xq, wq[:, ::-1]))  # k reversed
    assert _fails(test_hand_4x4_example)
    monkeypatch.setattr(O, "int8_gemm", orig_gemm)

    orig_dq = O.dequantize
    monkeypatch.setattr(O, "dequantize",
                        lambda acc, a, w, out: orig_dq(acc, np.asarray(a)[::-1].copy(), w, out))
    assert _fails(test_hand_4x4_example)
    monkeypatch.setattr(O, "dequantize", orig_dq)

    orig_shrink = O.lora_shrink
    monkeypatch.setattr(O, "lora_shrink", lambda x, dt, a: orig_shrink(x, "bf16", a) * 0)
    assert _fails(lambda: test_brute_force_lora(1))
    monkeypatch.setattr(O, "lora_shrink", orig_shrink)

    # segment bounds off by one: every request starts one row late (or early)
    orig_seg = O.lora_apply_segmented
    for shift in (1, -1):
        def seg_shifted(y, x, dt, seg_start, seg_adapter, A, B, scale, out, shift=shift):
            st = [min(max(int(v) + shift, 0), len(y)) if 0 < i < len(seg_start) - 1 else int(v)
                  for i, v in enumerate(seg_start)]
            return orig_seg(y, x, dt, st, seg_adapter, A, B, scale, out)
        monkeypatch.setattr(O, "lora_apply_segmented", seg_shifted)
        assert _fails(test_segmented_reduces_to_single_adapter)
    monkeypatch.setattr(O, "lora_apply_segmented", orig_seg)


def test_static_clip_count_brute_force_ties():
    """The clip count is the number of codes whose half-to-even rounding leaves
    [-127, 127] ("SmoothQuant" explainer, "How it works", Step 6, static scale):
    127.5 and 128.5 round to 128 and clip, 126.5 rounds to 126 and does not."""
    row = np.array([126.4, 127.4, 127.5, 128.6, -127.5, -127.49, 200.0, -1000.0,
                    126.5, 0.0, 1.0, -1.0, 127.0, -127.0, 128.5, 3.0], np.float32)
    x = np.stack([row, -row])
    q, clipped = O.quantize_per_tensor_static(x, None, np.float32(1.0))
    by_hand = 0
    for v in x.ravel():
        f = float(v)
        r = round(f)                      # Python rounds half to even
        by_hand += abs(r) > 127
    assert clipped == by_hand == 12
    assert q[0, 2] == 127 and q[0, 4] == -127 and q[0, 8] == 126 and q[0, 14] == 127
    # with a scale of 2 and s = 4 every value is divided by 8: nothing clips
    q8, c8 = O.quantize_per_tensor_static(x, np.full(16, 4.0, np.float32), np.float32(2.0))
    assert c8 == 0 and q8[0, 6] == 25
    # a zero scale gives zero codes and no clips
    q0, c0 = O.quantize_per_tensor_static(x, None, np.float32(0.0))
    assert c0 == 0 and not q0.any()


# ----------------------------------------------------------------------------
# Per-layer alpha search (R8)
# ----------------------------------------------------------------------------
def _brute_sweep_err(x, w, alpha, mode):
    """The same error with the pure-Python pipeline and exact rational sums."""
    from fractions import Fraction
    xl = [[float(v) for v in row] for row in x]
    wl = [[float(v) for v in row] for row in w]
    r = brute.pipeline(xl, wl, xl, alpha, mode=mode, out="f32")
    err = Fraction(0)
    ref = Fraction(0)
    for m in range(len(xl)):
        for n in range(len(wl)):
            yr = sum(Fraction(xl[m][k]) * Fraction(wl[n][k]) for k in range(len(xl[0])))
            d = Fraction(r["y32"][m][n]) - yr
            err += d * d
            ref += yr * yr
    return float(err), float(ref)


@pytest.mark.parametrize("mode", ["dynamic", "static"])
def test_alpha_sweep_matches_brute_force(mode):
    rng = np.random.default_rng(31)
    M, K, N = 4, 16, 5
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, [3, 11]] *= 40.0
    w = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    alphas = [0.0, 0.25, 0.5, 0.8, 1.0]
    sw = O.alpha_sweep(x, w, alphas, mode=mode)
    for i, a in enumerate(alphas):
        e, ref = _brute_sweep_err(x, w, a, mode)
        assert sw["ref"] == pytest.approx(ref, rel=1e-12)
        assert sw["err"][i] == pytest.approx(e, rel=1e-9), a
        assert sw["err"][i] > 0
    assert sw["best"] == alphas[int(np.argmin(sw["rel"]))]


@pytest.mark.parametrize("mode", ["dynamic", "static"])
def test_alpha_sweep_exact_layer_has_zero_error_at_half(mode):
    """A layer built from integer codes and power-of-two smoothing factors: at
    alpha = 0.5 the factors come out exactly, every division and scale is exact,
    the dequantized output equals the exact product and the error is 0. Other
    alphas give factors that are not powers of two, and nonzero error."""
    rng = np.random.default_rng(5)
    M, K, N = 6, 32, 7
    cx = rng.integers(-100, 101, (M, K))
    cw = rng.integers(-100, 101, (N, K))
    cx[np.arange(M), rng.integers(0, K, M)] = 127          # every row reaches 127
    cw[np.arange(N), rng.integers(0, K, N)] = -127
    # equal column maxima on both sides: c_k = max |cx[:, k]| = max |cw[:, k]|
    c = np.maximum(np.abs(cx).max(0), np.abs(cw).max(0))
    cx[0, :] = np.where(np.abs(cx).max(0) < c, c, cx[0, :])
    cw[0, :] = np.where(np.abs(cw).max(0) < c, c, cw[0, :])
    assert np.array_equal(np.abs(cx).max(0), np.abs(cw).max(0))
    assert (np.abs(cx).max(1) == 127).all() and (np.abs(cw).max(1) == 127).all()
    sk = np.exp2(rng.integers(-3, 4, K)).astype(np.float64)   # the smoothing factors
    x = (cx * sk).astype(np.float32)                          # a_k = c_k s_k
    w = (cw / sk).astype(np.float32)                          # w_k = c_k / s_k
    sw = O.alpha_sweep(x, w, [0.2, 0.5, 0.9], mode=mode)
    assert sw["err"][1] == 0.0
    assert sw["err"][0] > 0 and sw["err"][2] > 0
    assert sw["best"] == 0.5
    assert sw["ref"] == float(np.sum((cx.astype(np.float64) @ cw.T.astype(np.float64)) ** 2))


def test_alpha_sweep_scale_invariance_at_the_ends():
    """At alpha 0 and 1 the factors move by exact powers of two when X is scaled
    by 2, so every code is unchanged and the relative error is identical."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((8, 48)).astype(np.float32)
    x[:, 5] *= 30
    w = (rng.standard_normal((16, 48)) * 0.1).astype(np.float32)
    a = O.alpha_sweep(x, w, [0.0, 1.0])
    b = O.alpha_sweep(2 * x, w, [0.0, 1.0])
    assert np.array_equal(b["err"], 4 * a["err"]) and b["ref"] == 4 * a["ref"]
    assert np.array_equal(a["rel"], b["rel"])


# ----------------------------------------------------------------------------
# Normalization with the folded 1/s (R9)
# ----------------------------------------------------------------------------
def _norm_rows(seed, M=12, K=96):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((M, K)).astype(np.float32) * np.float32(3.0)
    h[:, [5, 40]] *= 50.0
    g = rng.uniform(0.5, 1.5, K).astype(np.float32)
    b = (rng.standard_normal(K) * 0.1).astype(np.float32)
    return h, g, b


@pytest.mark.parametrize("kind", ["rms", "layer"])
def test_norm_matches_torch_in_fp64(kind):
    """Unfolded (s = 1): the textbook normalizations, as torch computes them in fp64."""
    h, g, b = _norm_rows(1)
    eps = 1e-5
    ht, gt, bt = (torch.from_numpy(v).double() for v in (h, g, b))
    e = float(np.float32(eps))
    if kind == "rms":
        ref = torch.nn.functional.rms_norm(ht, (h.shape[1],), gt, eps=e).numpy()
        got = O.norm_smooth(h, "rms", g, None, eps)
    else:
        ref = torch.nn.functional.layer_norm(ht, (h.shape[1],), gt, bt, eps=e).numpy()
        got = O.norm_smooth(h, "layer", g, b, eps)
    assert got.dtype == np.float32
    np.testing.assert_allclose(got, ref, rtol=4e-7 * 4, atol=1e-6)


@pytest.mark.parametrize("kind", ["rms", "layer"])
def test_norm_fold_with_power_of_two_s_is_exact(kind):
    """With s a power of two, dividing g and b by s and dividing the norm output
    by s are both exact, so x_s * s is the unfolded normalization bit for bit."""
    h, g, b = _norm_rows(2)
    s = np.exp2(np.random.default_rng(3).integers(-4, 5, h.shape[1])).astype(np.float32)
    gf, bf = O.fold_norm_weight(g, b if kind == "layer" else None, s)
    xs = O.norm_smooth(h, kind, gf, bf, 1e-5)
    x = O.norm_smooth(h, kind, g, b if kind == "layer" else None, 1e-5)
    assert np.array_equal(xs * s, x)
    # and the smoothing direction: dividing x by s, not multiplying
    assert not np.array_equal(xs, x * s)


def test_norm_closed_forms():
    K = 64
    h = np.stack([np.full(K, 3.0, np.float32), np.full(K, -0.5, np.float32)])
    g = np.linspace(0.5, 2.0, K).astype(np.float32)
    b = np.linspace(-1.0, 1.0, K).astype(np.float32)
    mean, r = O.norm_stats(h, "rms", 1e-5)
    assert (mean == 0).all()
    assert r[0] == np.float32(1.0 / math.sqrt(9.0 + float(np.float32(1e-5))))
    # LayerNorm of a constant row: zero deviation, so the output is the bias
    xs = O.norm_smooth(h, "layer", g, b, 1e-5)
    assert np.array_equal(xs, np.stack([b, b]))
    mean, r = O.norm_stats(h, "layer", 1e-5)
    assert mean[0] == 3.0 and mean[1] == -0.5
    assert r[0] == np.float32(1.0 / math.sqrt(float(np.float32(1e-5))))
    # a row 0, 1, ..., K-1: mean (K-1)/2, biased variance (K^2 - 1)/12
    ramp = np.arange(K, dtype=np.float32)[None, :]
    mean, r = O.norm_stats(ramp, "layer", 0.0)
    assert mean[0] == (K - 1) / 2
    assert r[0] == np.float32(1.0 / math.sqrt((K * K - 1) / 12.0))


def test_norm_quant_codes_and_scales():
    h, g, b = _norm_rows(4)
    q, a, (mean, r) = O.norm_quant(h, "layer", g, b, 1e-5)
    xs = O.norm_smooth(h, "layer", g, b, 1e-5)
    for m in range(h.shape[0]):
        scale = brute.f32(max(abs(float(v)) for v in xs[m]) / 127.0)
        assert a[m] == np.float32(scale)
        assert list(q[m]) == brute.quant_row([float(v) for v in xs[m]], scale)
    # static: the given scale, clipping allowed
    qs, a_s, _ = O.norm_quant(h, "rms", g, None, 1e-5, mode="static", a_static=np.float32(0.01))
    assert a_s == np.float32(0.01) and np.abs(qs).max() == 127
