"""Exact-rational helpers for pins: round a rational to binary32 (nearest, ties to even)."""
from fractions import Fraction

import numpy as np


def bf16_fraction(bits):
    v = float((np.uint32(int(bits)) << np.uint32(16)).view(np.float32))
    return Fraction(v)


def rn_f32(r: Fraction) -> float:
    """Round a rational to the nearest binary32 value, ties to even (no overflow handling:
    callers stay in range).  Subnormal quantum 2^-149."""
    if r == 0:
        return 0.0
    neg = r < 0
    a = -r if neg else r
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    qexp = max(e - 23, -149)
    q = Fraction(2) ** qexp
    n = round(a / q)               # Fraction.__round__: half to even
    v = float(n * q)               # exact: n has <= 24 bits
    assert np.float32(v) == v
    return -v if neg else v
