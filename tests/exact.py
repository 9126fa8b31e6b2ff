"""Exact-rational helpers used to pin the oracle (test code only).

Rounding to an IEEE binary format is written out from its definition:
round-to-nearest, ties to the even significand, gradual underflow below the
smallest normal, overflow to infinity.  Everything is integer / Fraction
arithmetic, independent of numpy's and the FPU's rounding.
"""
from __future__ import annotations

import math
from fractions import Fraction

# (precision p incl. hidden bit, emin, emax)
BINARY32 = (24, -126, 127)
BINARY16 = (11, -14, 15)


def _floor_log2(a: Fraction) -> int:
    """e with 2**e <= a < 2**(e+1), for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_to_binary(v: Fraction, fmt=BINARY32) -> Fraction | float:
    """RN(v) in the binary format ``fmt``; returns a Fraction (or +-inf)."""
    p, emin, emax = fmt
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = max(_floor_log2(a), emin)           # below emin the quantum is fixed
    quantum = Fraction(2) ** (e - p + 1)
    n = a / quantum
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    r = lo * quantum
    largest = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if r > largest:
        return sign * math.inf
    return sign * r


def rn32(v: Fraction) -> Fraction | float:
    return round_to_binary(v, BINARY32)


def rn16(v: Fraction) -> Fraction | float:
    return round_to_binary(v, BINARY16)


def round_half_even_int(v: Fraction) -> int:
    lo = v.numerator // v.denominator
    rem = v - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return lo


def rn16_sqrt(v: Fraction) -> Fraction:
    """RN16(sqrt(v)) for a rational v >= 0, decided exactly.

    Candidates are the binary16 neighbours of an approximate root; the
    result is the one whose distance to sqrt(v) is smallest, compared
    through squares of midpoints (no irrational arithmetic).
    """
    if v == 0:
        return Fraction(0)
    approx = Fraction(math.sqrt(float(v)))
    c = rn16(approx)
    cands = {c}
    for _ in range(2):
        for x in list(cands):
            cands |= {binary_neighbour(x, +1, BINARY16), binary_neighbour(x, -1, BINARY16)}
    cands = sorted(x for x in cands if x >= 0 and x != math.inf)
    best = None
    for i, x in enumerate(cands):
        # x is the rounding of sqrt(v) iff sqrt(v) lies between the midpoints
        # to its neighbours (ties: even significand)
        lo_mid = (x + binary_neighbour(x, -1, BINARY16)) / 2 if x > 0 else Fraction(0)
        hi_mid = (x + binary_neighbour(x, +1, BINARY16)) / 2
        lo_ok = v > lo_mid * lo_mid or (v == lo_mid * lo_mid and _even16(x))
        hi_ok = v < hi_mid * hi_mid or (v == hi_mid * hi_mid and _even16(x))
        if lo_ok and hi_ok:
            best = x
    assert best is not None
    return best


def _even16(x: Fraction) -> bool:
    p, emin, _ = BINARY16
    e = max(_floor_log2(x), emin)
    return (x / Fraction(2) ** (e - p + 1)).numerator % 2 == 0


def binary_neighbour(x: Fraction, direction: int, fmt=BINARY32) -> Fraction:
    """The next representable value above (+1) or below (-1) x >= 0."""
    p, emin, _ = fmt
    if x == 0:
        q = Fraction(2) ** (emin - p + 1)
        return q if direction > 0 else -q
    e = max(_floor_log2(x), emin)
    q = Fraction(2) ** (e - p + 1)
    if direction < 0 and x == Fraction(2) ** e and e > emin:
        q = q / 2
    return x + direction * q
