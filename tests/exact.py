"""Exact-rational helpers for the oracle pins (tests only)."""

from fractions import Fraction

import numpy as np


def frac(x):
    """Exact rational value of a finite float32/float64."""
    return Fraction(float(x))


def rn32(q):
    """Round a Fraction to the nearest float32, ties to even (exact)."""
    if q == 0:
        return np.float32(0.0)
    f = np.float32(float(q))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]

    def key(c):
        return (abs(frac(c) - q), int(np.array(c, dtype=np.float32).view(np.uint32)) & 1)

    return np.float32(min(cands, key=key))


def round_half_even(q):
    """Nearest integer to a Fraction, ties to even."""
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def bf16_from_frac_rne(q32):
    """fp32 value -> bf16 bits by exact nearest-even rounding to 8 significant bits."""
    x = np.float32(q32)
    if x == 0:
        return int(np.array(x, dtype=np.float32).view(np.uint32)) >> 16
    q = frac(x)
    hi = np.array(x, dtype=np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    lo_c = np.array(hi, dtype=np.uint32).view(np.float32)
    up_bits = np.uint32(int(hi) + 0x10000)
    hi_c = np.array(up_bits, dtype=np.uint32).view(np.float32)
    d_lo = abs(frac(lo_c) - q)
    d_hi = abs(frac(hi_c) - q)
    if d_lo < d_hi or (d_lo == d_hi and ((int(hi) >> 16) & 1) == 0):
        return int(hi) >> 16
    return int(up_bits) >> 16
