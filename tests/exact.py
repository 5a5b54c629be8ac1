"""Exact rational arithmetic for pinning the oracle (test helper).

Everything here works on fractions.Fraction values and Python integers, independent of
both the oracle's C code and the GPU library: correctly rounded binary16 / binary32 by
search over the exact value sets, round-half-to-even, and brute-force code selection.
"""
from __future__ import annotations

import bisect
import math
from fractions import Fraction
from functools import lru_cache

import numpy as np


def frac(x) -> Fraction:
    """Exact value of a finite binary32/binary64 number."""
    return Fraction(float(x))


@lru_cache(maxsize=1)
def f16_table():
    """All non-negative finite binary16 values, ascending, with their bit patterns.

    Decoded from the format definition: bits e (5) and f (10); e = 0 gives f * 2^-24,
    otherwise (1024 + f) * 2^(e - 25)."""
    vals, bits = [], []
    for b in range(0, 0x7C00):
        e, f = b >> 10, b & 0x3FF
        v = Fraction(f, 1 << 24) if e == 0 else Fraction(1024 + f) * Fraction(2) ** (e - 25)
        vals.append(v)
        bits.append(b)
    return vals, bits


F16_MAX = Fraction(65504)


def rn_f16_bits(v: Fraction) -> int:
    """Bit pattern of the binary16 value nearest to v (ties to even bits; |v| >= 65520
    gives infinity)."""
    sign = 0x8000 if v < 0 else 0
    a = -v if v < 0 else v
    if a >= F16_MAX + 16:
        return sign | 0x7C00
    vals, bits = f16_table()
    i = bisect.bisect_left(vals, a)
    if i < len(vals) and vals[i] == a:
        return sign | bits[i]
    lo, hi = i - 1, i  # vals[lo] < a < vals[hi]
    if hi >= len(vals):
        return sign | bits[lo]
    dl, dh = a - vals[lo], vals[hi] - a
    if dl < dh:
        return sign | bits[lo]
    if dh < dl:
        return sign | bits[hi]
    return sign | (bits[lo] if bits[lo] % 2 == 0 else bits[hi])


def f16_value(b: int) -> Fraction:
    vals, _ = f16_table()
    v = vals[b & 0x7FFF]
    return -v if b & 0x8000 else v


def rn_f32(v: Fraction) -> Fraction:
    """Nearest binary32 value to v (ties to the even significand; gradual underflow)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = max(e - 23, -149)              # quantum of the binade (or of the subnormals)
    unit = Fraction(2) ** q
    m = a / unit
    n = math.floor(m)
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    out = n * unit
    if out >= Fraction(2) ** 128:
        raise OverflowError("binary32 overflow")
    return sign * out


def _f32_next(c: np.float32, up: bool) -> np.float32:
    return np.nextafter(c, np.float32(np.inf if up else -np.inf))


def rn_sqrt32(v: Fraction) -> Fraction:
    """Nearest binary32 value to sqrt(v), v > 0, decided exactly: the midpoint m between
    two neighbours satisfies sqrt(v) < m exactly when v < m * m."""
    c = np.float32(math.sqrt(float(v)))
    while True:
        nx = _f32_next(c, True)
        mid = (Fraction(float(c)) + Fraction(float(nx))) / 2
        if v > mid * mid or (v == mid * mid and (int(np.array([nx]).view(np.uint32)[0]) % 2 == 0)):
            c = nx
            continue
        pv = _f32_next(c, False)
        mid = (Fraction(float(pv)) + Fraction(float(c))) / 2
        if v < mid * mid or (v == mid * mid and (int(np.array([pv]).view(np.uint32)[0]) % 2 == 0)):
            c = pv
            continue
        return Fraction(float(c))


def rne_int(v: Fraction) -> int:
    n = math.floor(v)
    r = v - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def brute_code(x: Fraction, s: Fraction, Q: int) -> int:
    """argmin over every integer q in [-Q, Q] of |x/s - q|; among equals, the even one.
    This is the clamped round-half-to-even of x/s, found by enumeration."""
    best, bestd = None, None
    t = x / s
    for q in range(-Q, Q + 1):
        d = abs(t - q)
        if bestd is None or d < bestd or (d == bestd and q % 2 == 0):
            best, bestd = q, d
    return best


def kth_smallest_abs(xs, k: int) -> Fraction:
    return sorted(abs(x) for x in xs)[k - 1]


def ceil_rank(n: int, num: int, den: int) -> int:
    k = -((-num * n) // den)
    return min(max(k, 1), n)


def f32(x) -> np.float32:
    return np.float32(float(x))
