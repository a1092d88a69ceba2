"""Exact-arithmetic helpers for pinning the oracle (independent of it).

rn32() rounds an exact rational to IEEE binary32 (nearest, ties to even,
subnormals included) by integer arithmetic on Fractions, so it does not rely
on any floating-point unit.
"""
from __future__ import annotations

import struct
from fractions import Fraction

import numpy as np


def f32(x) -> float:
    """Python float holding exactly the binary32 value of x (x already binary32)."""
    return float(np.float32(x))


def rn32(x: Fraction) -> Fraction:
    """Round the rational x to the nearest binary32 value (ties to even)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                 # below that, the quantum is fixed (subnormals)
    quantum = Fraction(2) ** (e - 23)
    m = a / quantum                  # mantissa in units of the quantum
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r >= Fraction(2) ** 128 - Fraction(2) ** 103:   # beyond the largest finite value
        raise OverflowError("rn32 overflow")
    return sign * r


def rne_int(x: Fraction) -> int:
    """Round a rational to the nearest integer, ties to even."""
    fl = x.numerator // x.denominator
    rem = x - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return int(fl)


def as_frac(v) -> Fraction:
    return Fraction(float(v))


def f32_bits(v) -> int:
    return struct.unpack("<I", struct.pack("<f", float(v)))[0]


def bf16_bits_to_float(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(b) & 0xFFFF) << 16))[0]


def popcount(v: int) -> int:
    return bin(v).count("1")


def sylvester(n: int) -> np.ndarray:
    """Integer Sylvester-Hadamard matrix by the closed form (-1)^popcount(i & j)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    pc = np.vectorize(popcount)(i & j)
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)
