"""Independent vectorised emulation of the softmax-weight arithmetic.

Written from the definition (fp32 round-to-nearest-even for every step, fused
multiply-add rounded once), not from the oracle's C source.  numpy's float32
operations are IEEE round-to-nearest; the fused multiply-add is emulated in
float64 and every case where float64 rounding could have landed on a float32
tie is recomputed exactly with rationals, so the emulation is exact.
"""
from decimal import Decimal, getcontext
from fractions import Fraction
import math

import numpy as np

getcontext().prec = 80
_LN2 = Fraction(Decimal(2).ln())


def rn32_fraction(q: Fraction) -> float:
    """Round a rational to the nearest float32 (ties to even); normal range only."""
    if q == 0:
        return 0.0
    s = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    scaled = q * Fraction(2) ** (23 - e)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return float(s * n * Fraction(2) ** (e - 23))


L2E = np.float32(rn32_fraction(1 / _LN2))
COEF = [np.float32(rn32_fraction(_LN2 ** j / math.factorial(j))) for j in range(7)]


def _is_f32_midpoint(s: np.ndarray) -> np.ndarray:
    """True where a float64 value lies exactly halfway between two float32 values."""
    s = np.asarray(s, np.float64)
    bits = s.view(np.uint64)
    low = bits & np.uint64((1 << 29) - 1)          # the 29 mantissa bits float32 drops
    return (low == np.uint64(1 << 28)) & np.isfinite(s) & (s != 0)


def fma32(a, b, c) -> np.ndarray:
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    c = np.asarray(c, np.float32)
    a, b, c = np.broadcast_arrays(a, b, c)
    s = a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)
    out = s.astype(np.float32)
    mid = _is_f32_midpoint(s)
    if mid.any():
        for idx in zip(*np.nonzero(mid)):
            ex = Fraction(float(a[idx])) * Fraction(float(b[idx])) + Fraction(float(c[idx]))
            out[idx] = np.float32(rn32_fraction(ex))
    return out


def weights(l, M, T=1.0) -> np.ndarray:
    """floor(exp_spec(x) * 2^35) with x = (l - M) / T in float32; NaN propagates."""
    l = np.asarray(l, np.float32)
    x = (l - np.float32(M)).astype(np.float32)
    if T != 1.0:
        x = (x / np.float32(T)).astype(np.float32)
    isn = np.isnan(x)
    x = np.where(x < np.float32(-32.0), np.float32(-32.0), x).astype(np.float32)
    y = (x * L2E).astype(np.float32)
    n = np.rint(y).astype(np.float32)
    f = (y - n).astype(np.float32)
    p = np.full_like(f, COEF[6])
    for j in range(5, -1, -1):
        p = fma32(p, f, COEF[j])
    nn = np.where(isn, 0, n).astype(np.int64)
    e = np.ldexp(p.astype(np.float64), nn + 35)
    w = np.floor(e)
    w[isn] = np.nan
    return w


def exp_spec(x) -> np.ndarray:
    x = np.asarray(x, np.float32)
    x = np.where(x < np.float32(-32.0), np.float32(-32.0), x).astype(np.float32)
    y = (x * L2E).astype(np.float32)
    n = np.rint(y).astype(np.float32)
    f = (y - n).astype(np.float32)
    p = np.full_like(f, COEF[6])
    for j in range(5, -1, -1):
        p = fma32(p, f, COEF[j])
    return np.ldexp(p.astype(np.float64), n.astype(np.int64)).astype(np.float32)


def to_f32(a) -> np.ndarray:
    """float32 view of logits given as float32 or bf16 bits (uint16)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32)


def row_stats(row, C, T=1.0):
    """(M, W as python int, top ids, top weights as ints) for one row."""
    lf = to_f32(row)
    M = np.float32(np.max(lf))
    w = weights(lf, M, T)
    W = int(sum(int(v) for v in w))
    order = np.lexsort((np.arange(lf.size), -lf.astype(np.float64)))
    ids = order[:C]
    return M, W, ids, [int(w[i]) for i in ids]
