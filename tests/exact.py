"""Exact rational arithmetic for pinning the oracle's floating-point steps.

Nothing here calls the oracle or the library.  IEEE-754 binary32 rounding is
written out from its definition on ``fractions.Fraction`` values (round to
nearest, ties to even), so that a pin can state what a correctly rounded
float32 quotient or product is without computing it the way the oracle does.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

F32_MANT = 24          # significand bits of binary32, hidden bit included
F32_MIN_EXP = -149     # quantum of the subnormal range


def fr(x) -> Fraction:
    """The exact value of a float16/32/64 number."""
    return Fraction(float(x))


def round_half_even(x: Fraction) -> int:
    """The integer nearest x; halves go to the even neighbour."""
    q, r = divmod(x.numerator, x.denominator)          # x = q + r / den, 0 <= r < den
    twice = 2 * r
    if twice > x.denominator or (twice == x.denominator and q % 2):
        q += 1
    return q


def nearest_f32(x: Fraction) -> np.float32:
    """x rounded to the nearest binary32 value, ties to even (finite range)."""
    if x == 0:
        return np.float32(0.0)
    a = abs(x)
    # exponent e of the quantum: 2^(M-1) <= a / 2^e < 2^M for normal values
    e = a.numerator.bit_length() - a.denominator.bit_length() - F32_MANT
    while a >= Fraction(2) ** (e + F32_MANT):
        e += 1
    while a < Fraction(2) ** (e + F32_MANT - 1):
        e -= 1
    e = max(e, F32_MIN_EXP)
    m = round_half_even(a / Fraction(2) ** e)
    v = np.float32(m * 2.0 ** e)                      # exact: m <= 2^24
    assert fr(v) == m * Fraction(2) ** e
    return v if x > 0 else -v


def f32_tie_pairs(n: int, qmax: int, seed: int, scale_range=(1.0, 200.0)):
    """n pairs (x, s): s a float16 scale, x a float32 value, whose exact
    product is not a half-integer but whose float32 rounding is one, k + 1/2
    with |k + 1/2| < qmax.  Rounding the float32 product half-to-even and
    rounding the exact product to the nearest integer then give different
    codes whenever the exact product lies on the odd side of the tie."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        s = np.float16(rng.uniform(*scale_range))
        k = int(rng.integers(-qmax, qmax))
        t = Fraction(2 * k + 1, 2)
        if abs(t) >= qmax:
            continue
        x0 = nearest_f32(t / fr(s))
        for step in (0, 1, -1, 2, -2, 3, -3):
            x = x0
            for _ in range(abs(step)):
                x = np.nextafter(x, np.float32(np.inf if step > 0 else -np.inf), dtype=np.float32)
            p = fr(x) * fr(s)
            if p != t and fr(nearest_f32(p)) == t and round_half_even(t) != round_half_even(p):
                out.append((np.float32(x), s))
                break
    return out
