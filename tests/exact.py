"""Exact-arithmetic brute force used to pin the oracle.

Nothing here shares code with ``oracle/``: values are built from the e4m3fn
bit fields with integer arithmetic, fp32 rounding is done on exact
``fractions.Fraction`` values, and e4m3 rounding is a scan over all 127
non-negative codes. It is slow and only used on tiny inputs.
"""

from fractions import Fraction

import numpy as np


def e4m3_int512(code: int) -> int:
    """512 * value of a finite e4m3fn code, as an exact integer.

    Normal codes: (8 + m) * 2^(e - 10) * 512 = (8 + m) * 2^(e - 1);
    subnormal codes: (m / 8) * 2^-6 * 512 = m.
    """
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        raise ValueError("NaN code")
    mag = m if e == 0 else (8 + m) << (e - 1)
    return -mag if s else mag


E4M3_POS = [Fraction(e4m3_int512(c), 512) for c in range(0x7F)]  # codes 0x00..0x7E


def f32_round(x: Fraction) -> Fraction:
    """Round an exact rational to IEEE binary32, nearest-even, with subnormals."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)  # below 2^-126 the quantum stays 2^-149
    quantum = Fraction(2) ** (e - 23)
    q, r = divmod(a, quantum)
    if r * 2 > quantum or (r * 2 == quantum and q % 2 == 1):
        q += 1
    return sign * q * quantum


def e4m3_nearest(x: Fraction, negative: bool) -> int:
    """Brute-force nearest e4m3fn code to x (|x| <= 448), ties to even code."""
    a = abs(x)
    best, best_d = None, None
    for c, v in enumerate(E4M3_POS):
        d = abs(v - a)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best | (0x80 if negative else 0)


def quant_group_exact(xs):
    """(scale, codes) for one group of floats, by exact rational arithmetic."""
    fx = [Fraction(float(v)) for v in xs]
    neg = [bool(np.signbit(np.float32(v))) for v in xs]
    amax = max(abs(v) for v in fx)
    s = f32_round(amax / 448) if amax > 0 else Fraction(1)
    codes = []
    for v, n in zip(fx, neg):
        q = f32_round(v / s)
        q = max(min(q, Fraction(448)), Fraction(-448))
        codes.append(e4m3_nearest(q, n))
    return s, codes


def gemm_exact(a_q, a_s, w_q, w_s, rows=None, cols=None):
    """Exact C[m, n] as Fractions via integer group dot products.

    Each group sum is an exact integer in units of 2^-18 (int64 numpy
    products of the 512x-scaled codes); the fp32 scales enter as exact
    Fractions.
    """
    lut = np.array([e4m3_int512(c) if c not in (0x7F, 0xFF) else 0 for c in range(256)], dtype=np.int64)
    a_i = lut[np.asarray(a_q)]
    w_i = lut[np.asarray(w_q)]
    m, k = a_i.shape
    n = w_i.shape[0]
    g = k // 128
    if rows is None:
        pairs = [(i, j) for i in range(m) for j in range(n)]
    else:
        pairs = list(zip(rows, cols))
    out = []
    for i, j in pairs:
        sums = (a_i[i].reshape(g, 128) * w_i[j].reshape(g, 128)).sum(axis=1)
        tot = Fraction(0)
        for gi in range(g):
            tot += Fraction(float(a_s[i, gi])) * Fraction(float(w_s[j // 128, gi])) * int(sums[gi])
        out.append(tot / (1 << 18))
    return out


def gemm_w8a16_exact(a, w_q, w_s, rows=None, cols=None):
    """Exact C[m, n] as Fractions for a bf16 activation (given as floats) and
    block-FP8 weights: Fraction activation values times the 512x-scaled
    integer codes, per group, times the Fraction weight scale."""
    lut = [e4m3_int512(c) if c not in (0x7F, 0xFF) else 0 for c in range(256)]
    a = np.asarray(a, dtype=np.float64)
    w_q = np.asarray(w_q)
    m, k = a.shape
    n = w_q.shape[0]
    g = k // 128
    if rows is None:
        pairs = [(i, j) for i in range(m) for j in range(n)]
    else:
        pairs = list(zip(rows, cols))
    out = []
    for i, j in pairs:
        tot = Fraction(0)
        for gi in range(g):
            s = sum(Fraction(float(a[i, kk])) * lut[int(w_q[j, kk])] for kk in range(gi * 128, gi * 128 + 128))
            tot += Fraction(float(w_s[j // 128, gi])) * s
        out.append(tot / 512)
    return out
