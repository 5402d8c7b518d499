"""Pure-Python brute force of the SmoothQuant W8A8 path, for tiny inputs only.

An independent second reading of the same definitions, used to pin the
numpy oracle: Python ints for every integer sum, Python floats (fp64) with an
explicit rounding to fp32 after every fp32 operation, and the builtin round()
(half to even). It imports nothing from the oracle.

fp32 emulation: for +, *, / of two fp32 values, computing in fp64 and then
rounding once to fp32 gives the correctly rounded fp32 result, because fp64
carries more than 2*24+2 significand bits (no double-rounding error).
"""
from __future__ import annotations

import math
import struct
from decimal import Decimal, getcontext


def f32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


def bf16(x: float) -> float:
    """Round an fp32 value to bf16 (nearest, ties to even) by exact rational reasoning."""
    if x == 0.0:
        return x
    m, e = math.frexp(x)              # x = m * 2^e, 0.5 <= |m| < 1
    return math.ldexp(round(m * 256.0), e - 8)   # 8 significant bits, round() ties to even


def f16(x: float) -> float:
    return struct.unpack("<e", struct.pack("<e", x))[0]


def absmax_cols(rows):
    return [max(abs(r[k]) for r in rows) for k in range(len(rows[0]))]


def scale_s(a: float, w: float, alpha: float) -> float:
    a = max(a, 1e-5)
    w = max(w, 1e-5)
    if alpha == 0.5:
        s = math.sqrt(a) / math.sqrt(w)
    else:
        s = a ** alpha / w ** (1.0 - alpha)
    return f32(max(s, 1e-5))


def scale_s_decimal(a: float, w: float, alpha: float, digits: int = 50) -> float:
    """The exact value a^alpha / w^(1-alpha) to `digits` digits, then one fp32 rounding."""
    getcontext().prec = digits
    a = Decimal(max(a, 1e-5))
    w = Decimal(max(w, 1e-5))
    al = Decimal(alpha)
    v = (a.ln() * al).exp() / (w.ln() * (Decimal(1) - al)).exp()
    v = max(v, Decimal(1e-5))
    # Decimal -> nearest fp64 -> fp32. The fp64 step can only move a value that
    # sits within 2^-53 (relative) of an fp32 rounding boundary.
    return f32(float(v))


def quant_row(vals, scale):
    if scale == 0.0:
        return [0 for _ in vals]
    return [max(-127, min(127, round(f32(v / scale)))) for v in vals]


def pipeline(x, w, x_cal, alpha, mode="dynamic", out="bf16"):
    """x [M][K], w [N][K], x_cal [C][K] as lists of fp32-exact floats."""
    M, K, N = len(x), len(x[0]), len(w)
    act_max = absmax_cols(x_cal)
    w_max = absmax_cols(w)
    s = [scale_s(act_max[k], w_max[k], alpha) for k in range(K)]
    ws = [[f32(w[n][k] * s[k]) for k in range(K)] for n in range(N)]
    w_scale = [f32(max(abs(v) for v in ws[n]) / 127.0) for n in range(N)]
    wq = [quant_row(ws[n], w_scale[n]) for n in range(N)]
    xs = [[f32(x[m][k] / s[k]) for k in range(K)] for m in range(M)]
    if mode == "dynamic":
        a_scale = [f32(max(abs(v) for v in xs[m]) / 127.0) for m in range(M)]
    else:
        st = f32(max(f32(act_max[k] / s[k]) for k in range(K)) / 127.0)
        a_scale = [st] * M
    xq = [quant_row(xs[m], a_scale[m]) for m in range(M)]
    acc = [[sum(xq[m][k] * wq[n][k] for k in range(K)) for n in range(N)] for m in range(M)]
    y32 = [[f32(f32(f32(float(acc[m][n])) * a_scale[m]) * w_scale[n]) for n in range(N)]
           for m in range(M)]
    rnd = {"bf16": bf16, "f16": f16, "f32": lambda v: v}[out]
    y = [[rnd(v) for v in row] for row in y32]
    return dict(act_max=act_max, w_max=w_max, s=s, ws=ws, w_scale=w_scale, wq=wq, xs=xs,
                a_scale=a_scale, xq=xq, acc=acc, y32=y32, y=y)


def lora(y, x, a, b, scale, x_is_bf16=True, out="bf16"):
    """Y = out(y + scale * bf16(bf16(x) A^T) B^T); sums exact (Fractions via floats' exactness
    would be overkill: tiny shapes, fp64 sums of bf16 products are exact enough)."""
    from fractions import Fraction
    M, K, r, N = len(x), len(x[0]), len(a), len(b)
    xb = x if x_is_bf16 else [[bf16(v) for v in row] for row in x]
    t = [[bf16(float(sum(Fraction(xb[m][k]) * Fraction(a[i][k]) for k in range(K))))
          for i in range(r)] for m in range(M)]
    rnd = {"bf16": bf16, "f16": f16, "f32": f32}[out]
    res = []
    for m in range(M):
        row = []
        for n in range(N):
            d = sum(Fraction(t[m][i]) * Fraction(b[n][i]) for i in range(r))
            row.append(rnd(float(Fraction(y[m][n]) + Fraction(scale) * d)))
        res.append(row)
    return t, res
