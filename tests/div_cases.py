"""Hard inputs for the exact fp32 divisions of the quantizer (test input
construction only).

near_midpoint_pairs(n, seed) returns fp32 pairs (x, d) whose exact quotient
x / d lies within about 2^-48 (relative) of an fp32 rounding midpoint, on
either side of it: the cases where any approximate division path rounds the
wrong way first. Construction: d = D 2^-23 with D odd in [2^23, 2^24); a
midpoint in [0.5, 1) is m = A 2^-25 with A odd in [2^24, 2^25); picking
A = r D^-1 (mod 2^25) for a small odd r makes A D - r a multiple of 2^25,
k = (A D - r) / 2^25 < 2^24, so x = k 2^-23 is an fp32 number and
x / d = m - r 2^-25 / D. x is then scaled by 2^e and given a random sign.
"""
from __future__ import annotations

import numpy as np


def near_midpoint_pairs(n: int, seed: int, exp_range: int = 6):
    rng = np.random.default_rng(seed)
    m25 = 1 << 25
    xs, ds, rs = [], [], []
    while len(xs) < n:
        D = int(rng.integers(1 << 22, 1 << 23)) * 2 + 1
        Dinv = pow(D, -1, m25)
        for r in (1, -1, 3, -3, 5, -5, 7, -7):
            A = (r * Dinv) % m25
            if A < (1 << 24):
                continue
            k, rem = divmod(A * D - r, m25)
            assert rem == 0 and 0 < k < (1 << 24)
            e = int(rng.integers(-exp_range, exp_range + 1))
            sign = -1.0 if rng.random() < 0.5 else 1.0
            xs.append(sign * np.ldexp(float(k), e - 23))
            ds.append(np.ldexp(float(D), -23))
            rs.append(r)
            break
    return np.array(xs, np.float32), np.array(ds, np.float32), np.array(rs)
