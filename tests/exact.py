"""Exact rational helpers for pinning the oracle (tests only).

They round a Python Fraction to binary32 or bfloat16 by exact integer
arithmetic, independently of numpy's and torch's own rounding code.
"""
from fractions import Fraction

import numpy as np


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # bring e to floor(log2(a)): 2^e <= a < 2^(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_fraction(fr: Fraction, sig_bits: int, emin: int = -126) -> Fraction:
    """Nearest value (ties to even) with `sig_bits` significant bits and
    minimum normal exponent `emin` (subnormals have the fixed spacing
    2^(emin - sig_bits + 1)).  No overflow handling."""
    fr = Fraction(fr)
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - (sig_bits - 1))
    k = a / quantum
    fl = k.numerator // k.denominator
    rem = k - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def f32_of(fr: Fraction) -> np.float32:
    """Fraction -> nearest binary32 (as np.float32)."""
    return np.float32(float(round_fraction(fr, 24)))


def bf16_bits_of(fr: Fraction) -> int:
    """Fraction -> nearest bfloat16, as its 16-bit pattern (+0 for zero)."""
    v = np.float32(float(round_fraction(fr, 8)))
    bits = int(np.array([v], np.float32).view(np.uint32)[0] >> 16)
    if fr < 0 and v == 0:
        bits |= 0x8000
    return bits


def exact_quotient_f32(a: np.float32, m: np.float32) -> Fraction:
    """The binary32 quotient a / m (round to nearest even), as a Fraction."""
    return Fraction(float(round_fraction(Fraction(float(a)) / Fraction(float(m)), 24)))
