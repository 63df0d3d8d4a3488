"""Exact-rational model of the binary32 group quantizer (test aid).

Each step of the quantizer is modelled as the exact rational result followed
by an explicit round-to-nearest-even onto the binary32 grid.  This uses only
Python integers and fractions, no floating-point hardware, so it checks the
oracle's compiled float code by an independent mechanism: a contracted
multiply-add, a double rounding, a reciprocal in place of a divide or a
different rounding rule would each show up as a code mismatch.
"""
from fractions import Fraction

_TWO = Fraction(2)


def _floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # adjust so that 2^e <= a < 2^(e+1)
    while _TWO ** e > a:
        e -= 1
    while _TWO ** (e + 1) <= a:
        e += 1
    return e


def round_half_even(x: Fraction) -> int:
    """Nearest integer, ties to even."""
    fl = x.numerator // x.denominator
    rem = x - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def rn32(x: Fraction) -> Fraction:
    """Round an exact rational to the nearest binary32 value (ties to even).
    Values beyond the binary32 range are not expected here."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = _floor_log2(a)
    quantum = _TWO ** (max(e, -126) - 23)  # subnormals share 2^-149
    n = round_half_even(a / quantum)
    return sign * n * quantum


def quantize_group_exact(xs, bits):
    """xs: exact rationals (values of fp16/bf16/fp32 inputs).
    Returns (codes, s) with s the binary32 scale as a rational."""
    qmax = (1 << bits) - 1
    mn, mx = min(xs), max(xs)
    s = rn32(rn32(mx - mn) / qmax)
    if s == 0:
        return [0] * len(xs), s
    codes = []
    for x in xs:
        d = rn32(x - mn)
        y = rn32(d / s)
        c = round_half_even(y)
        codes.append(min(max(c, 0), qmax))
    return codes, s
