"""CPU oracle for the SmoothQuant W8A8 linear path with a bf16 LoRA delta.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or call this module. The product path
(the HIP library and its Python binding) never touches it, and this module
shares no code with that path.

It is deliberately plain and slow: numpy arrays, one step per function, in
the order the pages give them, with the floating-point precision of every
operation written out. Where the pages leave a point open, the reading taken
is stated at the function that uses it.

Sources (page titles and sections):
  [SQ]   "SmoothQuant" explainer (ozercemkelahmet.com/tools/smoothquant):
         "How it works" Steps 2-7, "A worked example", "A short Python
         sketch", "Calibration in practice".
  [LoRA] TensorRT-LLM issue #12703 "LoRA support for W8A8 SmoothQuant
         (SmoothQuantAttention / SmoothQuantLinear)", section "Pitch".
  [GRP]  TensorRT-LLM PR #17521 "Add FP8 LoRA support for B200",
         "Description" (per-request adapters in one grouped GEMM).

Readings of points the pages leave open (each used below):
  R1 weight layout: W is [N, K] (out_features, in_features), as in the
     sketch's nn.Linear convention, not the [K, N] of Step 1.
  R2 the smoothing scale s is evaluated in fp64 (sqrt form when alpha is
     exactly 0.5) and rounded once to fp32; the three 1e-5 clamps of the
     sketch are kept, as fp64 constants.
  R3 the divide by s and by the quantization scale are IEEE fp32 divisions
     (the sketch writes both as divisions); rounding is half-to-even on the
     fp32 quotient (torch.round in the sketch); codes are clamped to
     [-127, 127] (symmetric; the sketch's -128 is never reached by a
     dynamic absmax scale).
  R4 a row (or weight row) whose absmax is zero gets scale 0 and codes 0.
  R5 dequant is (fp32(acc) * a_scale[m]) * w_scale[n], left to right in fp32,
     then one round-to-nearest-even to the output dtype.
  R6 LoRA reads the original (unsmoothed) input rounded to bf16; the rank-r
     intermediate T is rounded to bf16; the delta (times a caller-given scale,
     1.0 by default) is added to the already-rounded GEMM output and rounded
     once more to the output dtype.
  R7 a static per-tensor activation scale is max_k(act_max_cal[k] / s[k]) /
     127 from the calibration batch, i.e. the sketch's per-tensor absmax of
     the smoothed calibration activations.
  R8 the per-layer alpha search ("Calibration in practice": pick the
     migration strength per layer by how well the quantized layer reproduces
     its output on calibration data) measures, for each candidate alpha, the
     squared error of the fp32 dequantized output against the exact
     unquantized output X W^T on the calibration batch itself (which also
     supplies the activation maxima), relative to the squared norm of that
     output. The output is compared before any rounding to a 16-bit output
     type, so the error is the quantization error alone.
  R9 the normalization before a projection ("How it works", Step 5: the
     division by s can ride on the preceding normalization's weight; the
     sketch divides the norm weight and bias by s) uses the textbook
     definitions: RMSNorm x = h / sqrt(mean(h^2) + eps) * g, LayerNorm
     x = (h - mean(h)) / sqrt(var(h) + eps) * g + b (biased variance). The
     folded weight and bias g / s, b / s are single fp32 divisions. Row
     statistics: sums taken exactly (correctly rounded fp64 sums), the mean
     rounded to fp32, h - mean rounded to fp32, the inverse root
     1 / sqrt(. + eps) evaluated in fp64 and rounded to fp32. Then
     x_s = fp32(fp32(h * r) * g') (RMS) or
     x_s = fp32(fp32(fp32((h - mean) * r) * g') + b') (LayerNorm), quantized
     per token (or with a static scale) exactly as x_s from Step 5.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

F32 = np.float32
QMAX = 127           # R3: symmetric INT8 range [-127, 127]
CLAMP_MIN = 1e-5     # R2: the sketch's clamp(min=1e-5), as an fp64 constant


# ----------------------------------------------------------------------------
# Rounding to the 16-bit storage types (round to nearest, ties to even).
# ----------------------------------------------------------------------------
def round_f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (RNE), returned as fp32 values that are exactly bf16.

    bf16 keeps the top 16 bits of an fp32 word. Adding 0x7FFF plus the lowest
    kept bit before truncating rounds to nearest with ties to even.
    Finite inputs only.
    """
    b = np.ascontiguousarray(x, dtype=F32).view(np.uint32).astype(np.uint64)
    keep_lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = ((b + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(F32).reshape(np.shape(x))


def round_f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 with one RNE rounding (no intermediate fp32 rounding).

    x = m * 2**e with 0.5 <= |m| < 1; bf16 keeps 8 significant bits, so the
    value is rint(m * 2**8) * 2**(e - 8). Valid for the normal bf16 range,
    which is the only range these workloads reach.
    """
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8).astype(F32)


def to_out_dtype(y: np.ndarray, out_dtype: str) -> np.ndarray:
    """Round fp32 or fp64 values to the output dtype (RNE).

    Returns fp32 for 'f32' and 'bf16' (bf16 values held in fp32) and
    float16 for 'f16'.
    """
    y = np.asarray(y)
    if out_dtype == "f32":
        return y.astype(F32)
    if out_dtype == "f16":
        return y.astype(np.float16)          # numpy rounds directly to half, RNE
    if out_dtype == "bf16":
        return round_f64_to_bf16(y) if y.dtype == np.float64 else round_f32_to_bf16(y)
    raise ValueError(out_dtype)


# ----------------------------------------------------------------------------
# [SQ] Step 4 and "Calibration in practice": per-channel activation maxima.
# ----------------------------------------------------------------------------
def calibrate_absmax(x: np.ndarray, act_max: Optional[np.ndarray] = None) -> np.ndarray:
    """Running per-input-channel max of |x| over the rows of a calibration batch.

    x: [rows, K] fp32 values (exact widening of the input dtype).
    act_max: previous running max [K] (fp32) or None. Max is exact in fp32.
    """
    m = np.abs(np.asarray(x, dtype=F32)).max(axis=0) if len(x) else np.zeros(x.shape[1], F32)
    return m if act_max is None else np.maximum(np.asarray(act_max, F32), m)


# ----------------------------------------------------------------------------
# [SQ] Step 3 and the sketch's smooth_layer: the smoothing scale.
# ----------------------------------------------------------------------------
def weight_absmax(w: np.ndarray) -> np.ndarray:
    """max over output rows of |W[n, k]| for each input channel k (R1: W is [N, K])."""
    return np.abs(np.asarray(w, dtype=F32)).max(axis=0)


def smoothing_scale(act_max: np.ndarray, w_max: np.ndarray, alpha: float) -> np.ndarray:
    """s_k = max(a_k, 1e-5)^alpha / max(w_k, 1e-5)^(1 - alpha), clamped below at 1e-5.

    R2: fp64 evaluation, one rounding to fp32. At alpha == 0.5 the two powers
    are square roots, taken with sqrt (correctly rounded) rather than pow.
    """
    a = np.maximum(np.asarray(act_max, np.float64), CLAMP_MIN)
    w = np.maximum(np.asarray(w_max, np.float64), CLAMP_MIN)
    alpha = float(alpha)
    if alpha == 0.5:
        s = np.sqrt(a) / np.sqrt(w)
    else:
        s = np.power(a, alpha) / np.power(w, 1.0 - alpha)
    return np.maximum(s, CLAMP_MIN).astype(F32)


# ----------------------------------------------------------------------------
# [SQ] Step 6 and the sketch's quantize_int8: symmetric absmax quantization.
# ----------------------------------------------------------------------------
def quantize_rows(t: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """q = clamp(rne(fp32(t / scale)), -127, 127); rows with scale 0 give 0 (R3, R4)."""
    t = np.asarray(t, F32)
    scale = np.asarray(scale, F32).reshape(-1, 1) if np.ndim(scale) else np.asarray(scale, F32)
    q = np.zeros(t.shape, np.int8)
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = t / scale                                   # fp32 / fp32 -> fp32
    ok = np.broadcast_to(scale != 0, t.shape)
    q[ok] = np.clip(np.rint(quot[ok]), -QMAX, QMAX).astype(np.int8)
    return q


def row_absmax_scale(t: np.ndarray) -> np.ndarray:
    """Per-row scale max_k |t[r, k]| / 127 in fp32 (the sketch's per-channel amax / 127)."""
    t = np.asarray(t, F32)
    amax = np.abs(t).max(axis=1) if t.shape[1] else np.zeros(t.shape[0], F32)
    return amax / F32(QMAX)


# ----------------------------------------------------------------------------
# [SQ] Step 5 (fold s into the weight columns) + Step 6 (per-output-channel).
# ----------------------------------------------------------------------------
def fold_and_quantize_weights(w: np.ndarray, s: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """W_s[n, k] = fp32(W[n, k] * s[k]); per output row: w_scale = absmax / 127, Wq codes.

    Returns (Wq [N, K] int8, w_scale [N] fp32).
    """
    ws = np.asarray(w, F32) * np.asarray(s, F32)[None, :]          # fp32 multiply
    w_scale = row_absmax_scale(ws)
    return quantize_rows(ws, w_scale), w_scale


# ----------------------------------------------------------------------------
# [SQ] Step 5 (divide the layer input by s) + Step 6 (per-token, dynamic or static).
# ----------------------------------------------------------------------------
def smooth_activations(x: np.ndarray, s: Optional[np.ndarray]) -> np.ndarray:
    """x_s[m, k] = fp32(x[m, k] / s[k]) (R3); no smoothing when s is None."""
    x = np.asarray(x, F32)
    return x if s is None else x / np.asarray(s, F32)[None, :]


def quantize_per_token(x: np.ndarray, s: Optional[np.ndarray]) -> Tuple[np.ndarray, np.ndarray]:
    """Dynamic per-token quantization of the smoothed input. Returns (Xq [M,K], a_scale [M])."""
    xs = smooth_activations(x, s)
    a_scale = row_absmax_scale(xs)
    return quantize_rows(xs, a_scale), a_scale


def static_activation_scale(act_max_cal: np.ndarray, s: Optional[np.ndarray]) -> np.float32:
    """R7: one per-tensor scale from calibration maxima: max_k fp32(a_k / s_k) / 127."""
    a = np.asarray(act_max_cal, F32)
    sm = a if s is None else a / np.asarray(s, F32)
    return F32(sm.max() / F32(QMAX))


def quantize_per_tensor_static(x: np.ndarray, s: Optional[np.ndarray],
                               a_scale: np.float32) -> Tuple[np.ndarray, int]:
    """Static per-tensor quantization with a fixed scale; values beyond it clip.

    Returns (Xq [M, K], number of clipped elements).
    """
    xs = smooth_activations(x, s)
    q = quantize_rows(xs, np.full(xs.shape[0], a_scale, F32))
    with np.errstate(divide="ignore", invalid="ignore"):
        clipped = int(np.count_nonzero(np.abs(np.rint(xs / F32(a_scale))) > QMAX)) if a_scale else 0
    return q, clipped


# ----------------------------------------------------------------------------
# [SQ] Step 7: INT8 x INT8 -> INT32 products, then dequant with stored scales.
# ----------------------------------------------------------------------------
def int8_gemm(xq: np.ndarray, wq: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k Xq[m, k] * Wq[n, k], exact, returned as int32.

    The sum is formed with a float64 matrix product. Every product is an
    integer of magnitude at most 127^2 and every partial sum an integer of
    magnitude at most K * 127^2 < 2^53, so each float64 operation (including
    fused multiply-adds) is exact and the result equals the integer sum.
    """
    xq = np.asarray(xq, np.int8)
    wq = np.asarray(wq, np.int8)
    K = xq.shape[1]
    assert K * QMAX * QMAX < 2 ** 53
    acc = xq.astype(np.float64) @ wq.astype(np.float64).T
    acc = acc.astype(np.int64)
    assert np.all(np.abs(acc) < 2 ** 31), "accumulator exceeds int32"
    return acc.astype(np.int32)


def dequantize(acc: np.ndarray, a_scale, w_scale: np.ndarray, out_dtype: str) -> np.ndarray:
    """R5: y = out_dtype((fp32(acc) * a_scale[m]) * w_scale[n]).

    a_scale is [M] (per token) or a scalar (per tensor).
    """
    af = np.asarray(acc).astype(F32)                     # int32 -> fp32, RNE
    a = np.asarray(a_scale, F32)
    a = a.reshape(-1, 1) if a.ndim else a
    y = (af * a) * np.asarray(w_scale, F32)[None, :]
    return to_out_dtype(y, out_dtype)


# ----------------------------------------------------------------------------
# [LoRA] Pitch: low-rank path in bf16 after the INT8 GEMM, added to its output.
# ----------------------------------------------------------------------------
def lora_shrink(x: np.ndarray, in_dtype: str, a: np.ndarray) -> np.ndarray:
    """T[m, i] = bf16(sum_k bf16(x[m, k]) * A[i, k]), sum in fp64 (R6). A is [r, K] bf16."""
    xb = np.asarray(x, F32) if in_dtype == "bf16" else round_f32_to_bf16(x)
    t = xb.astype(np.float64) @ np.asarray(a, np.float64).T
    return round_f64_to_bf16(t)


def lora_expand_add(y: np.ndarray, t: np.ndarray, b: np.ndarray, scale: float,
                    out_dtype: str) -> np.ndarray:
    """Y[m, n] = out_dtype(y[m, n] + scale * sum_i T[m, i] * B[n, i]) in fp64 (R6)."""
    d = np.asarray(t, np.float64) @ np.asarray(b, np.float64).T
    return to_out_dtype(np.asarray(y, np.float64) + float(scale) * d, out_dtype)


def lora_apply(y: np.ndarray, x: np.ndarray, in_dtype: str, a: np.ndarray, b: np.ndarray,
               scale: float, out_dtype: str) -> np.ndarray:
    return lora_expand_add(y, lora_shrink(x, in_dtype, a), b, scale, out_dtype)


def lora_apply_segmented(y: np.ndarray, x: np.ndarray, in_dtype: str,
                         seg_start: Sequence[int], seg_adapter: Sequence[int],
                         adapters_a: Sequence[np.ndarray], adapters_b: Sequence[np.ndarray],
                         scale: float, out_dtype: str) -> np.ndarray:
    """[GRP] one adapter per request: rows [seg_start[g], seg_start[g+1]) use adapter
    seg_adapter[g]; adapter -1 leaves those rows as they are."""
    y = np.array(y, copy=True)
    for g in range(len(seg_adapter)):
        r0, r1, ad = int(seg_start[g]), int(seg_start[g + 1]), int(seg_adapter[g])
        if ad < 0 or r1 <= r0:
            continue
        y[r0:r1] = lora_apply(y[r0:r1], x[r0:r1], in_dtype, adapters_a[ad], adapters_b[ad],
                              scale, out_dtype)
    return y


# ----------------------------------------------------------------------------
# The whole path for one input feeding one or more projections.
# ----------------------------------------------------------------------------
def smoothquant_linear(x: np.ndarray, in_dtype: str, w: np.ndarray, x_cal: np.ndarray,
                       alpha: float, out_dtype: str, mode: str = "dynamic",
                       lora: Optional[Tuple[np.ndarray, np.ndarray, float]] = None) -> dict:
    """Calibrate on x_cal, smooth and fold into W, quantize x, INT8 GEMM, dequant, LoRA.

    Returns every intermediate so each stage can be compared on its own.
    """
    act_max = calibrate_absmax(x_cal)
    w_max = weight_absmax(w)
    s = smoothing_scale(act_max, w_max, alpha)
    wq, w_scale = fold_and_quantize_weights(w, s)
    out = {"act_max": act_max, "w_max": w_max, "s": s, "wq": wq, "w_scale": w_scale}
    if mode == "dynamic":
        xq, a_scale = quantize_per_token(x, s)
        out["clipped"] = 0
    else:
        a_scale = static_activation_scale(act_max, s)
        xq, out["clipped"] = quantize_per_tensor_static(x, s, a_scale)
    acc = int8_gemm(xq, wq)
    y = dequantize(acc, a_scale, w_scale, out_dtype)
    out.update(xq=xq, a_scale=a_scale, acc=acc, y=y)
    if lora is not None:
        a, b, sc = lora
        out["y_lora"] = lora_apply(y, x, in_dtype, a, b, sc, out_dtype)
    return out


# ----------------------------------------------------------------------------
# [SQ] "Calibration in practice": per-layer choice of the migration strength.
# ----------------------------------------------------------------------------
def alpha_sweep(x_cal: np.ndarray, w: np.ndarray, alphas: Sequence[float],
                mode: str = "dynamic") -> dict:
    """R8: for each alpha, run the whole W8A8 path on the calibration batch and
    measure its output error against the unquantized layer.

    x_cal [M, K] and w [N, K] hold the exact input values (fp32 arrays).
    Returns err[i] = sum (y_i - y_ref)^2 and ref = sum y_ref^2 (fp64), with
    y_i the fp32 dequantized output at alphas[i] and y_ref = x_cal w^T in
    fp64; rel[i] = err[i] / ref; best = the alpha of the smallest rel (the
    first one on ties).
    """
    y_ref = np.asarray(x_cal, np.float64) @ np.asarray(w, np.float64).T
    ref = float(np.sum(y_ref * y_ref))
    err = []
    for a in alphas:
        r = smoothquant_linear(x_cal, "f32", w, x_cal, float(a), "f32", mode=mode)
        d = r["y"].astype(np.float64) - y_ref
        err.append(float(np.sum(d * d)))
    err = np.array(err, np.float64)
    rel = err / ref if ref > 0 else np.zeros_like(err)
    return {"err": err, "ref": ref, "rel": rel, "best": float(alphas[int(np.argmin(rel))])}


# ----------------------------------------------------------------------------
# [SQ] "How it works", Step 5 and the sketch's smooth_layer: 1/s folded into
# the normalization that precedes the projection, then per-token quant.
# ----------------------------------------------------------------------------
def fold_norm_weight(gamma: np.ndarray, beta: Optional[np.ndarray],
                     s: np.ndarray) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """R9: g' = fp32(g / s), b' = fp32(b / s) (IEEE fp32 divisions)."""
    s = np.asarray(s, F32)
    g = np.asarray(gamma, F32) / s
    b = None if beta is None else np.asarray(beta, F32) / s
    return g, b


def norm_stats(h: np.ndarray, kind: str, eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """R9: per-row (mean, inverse root) in fp32. kind: 'rms' (mean 0) or 'layer'."""
    h = np.asarray(h, F32)
    M, K = h.shape
    e = float(F32(eps))
    mean = np.zeros(M, F32)
    r = np.zeros(M, F32)
    for m in range(M):
        row = h[m].astype(np.float64)
        if kind == "layer":
            mean[m] = F32(math.fsum(row) / K)
            d = (h[m] - mean[m]).astype(np.float64)          # fp32 subtraction, widened
            ms = math.fsum(d * d) / K                        # products exact in fp64
        else:
            ms = math.fsum(row * row) / K
        r[m] = F32(1.0 / math.sqrt(ms + e))
    return mean, r


def norm_smooth(h: np.ndarray, kind: str, g_fold: np.ndarray, b_fold: Optional[np.ndarray],
                eps: float, stats: Optional[Tuple[np.ndarray, np.ndarray]] = None) -> np.ndarray:
    """R9: the smoothed activations x_s straight from the residual stream h."""
    h = np.asarray(h, F32)
    mean, r = norm_stats(h, kind, eps) if stats is None else stats
    g = np.asarray(g_fold, F32)[None, :]
    if kind == "layer":
        d = h - np.asarray(mean, F32)[:, None]
        x = (d * np.asarray(r, F32)[:, None]) * g
        return x + np.asarray(b_fold, F32)[None, :] if b_fold is not None else x
    return (h * np.asarray(r, F32)[:, None]) * g


def norm_quant(h: np.ndarray, kind: str, g_fold: np.ndarray, b_fold: Optional[np.ndarray],
               eps: float, mode: str = "dynamic", a_static=None,
               stats: Optional[Tuple[np.ndarray, np.ndarray]] = None):
    """Normalization with the folded weight, then INT8 codes.

    Returns (Xq, a_scale, (mean, r)); a_scale is [M] (dynamic) or the given
    static scale. `stats` replaces the row statistics (to check codes given
    another implementation's statistics)."""
    st = norm_stats(h, kind, eps) if stats is None else stats
    xs = norm_smooth(h, kind, g_fold, b_fold, eps, st)
    if mode == "dynamic":
        a = row_absmax_scale(xs)
        return quantize_rows(xs, a), a, st
    q, _ = quantize_per_tensor_static(xs, None, F32(a_static))
    return q, F32(a_static), st
