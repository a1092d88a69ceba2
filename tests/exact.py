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


# ----------------------------------------------------------------------------
# High-precision activations (Python decimal), for pinning the oracle's
# input activations independently of any libm.

import decimal as _dec

_CTX = _dec.Context(prec=70, Emax=10 ** 7, Emin=-10 ** 7)


def _atan_inv(n: int) -> _dec.Decimal:
    """atan(1/n) by its Taylor series."""
    with _dec.localcontext(_CTX):
        x = _dec.Decimal(1) / n
        x2 = x * x
        term, total, k = x, x, 1
        while True:
            term = -term * x2
            add = term / (2 * k + 1)
            if abs(add) < _dec.Decimal(10) ** -75:
                return total
            total += add
            k += 1


def dec_pi() -> _dec.Decimal:
    """pi by Machin's formula 16 atan(1/5) - 4 atan(1/239)."""
    with _dec.localcontext(_CTX):
        return 16 * _atan_inv(5) - 4 * _atan_inv(239)


_PI = dec_pi()


def dec_erfc(z: _dec.Decimal) -> _dec.Decimal:
    """erfc(z): Taylor series of erf for |z| <= 6, continued fraction beyond."""
    with _dec.localcontext(_CTX):
        if z < 0:
            return 2 - dec_erfc(-z)
        if z <= 6:
            z2 = z * z
            term, total, n = z, z, 0
            while True:
                n += 1
                term = -term * z2 / n
                add = term / (2 * n + 1)
                total += add
                if abs(add) < _dec.Decimal(10) ** -68:
                    break
            return 1 - 2 / _PI.sqrt() * total
        if z * z > 10 ** 6:
            return _dec.Decimal(0)
        # erfc(z) = e^{-z^2}/sqrt(pi) / (z + (1/2)/(z + 1/(z + (3/2)/(z + ...)))), evaluated backwards
        t = z
        for n in range(2000, 0, -1):
            t = z + (_dec.Decimal(n) / 2) / t
        return (-(z * z)).exp() / _PI.sqrt() / t


def dec_act(act: int, x: float):
    """The activation at x as a Decimal (None for 'rounds to zero with x's sign')."""
    with _dec.localcontext(_CTX):
        d = _dec.Decimal(x)
        if act == 1:                                  # GELU, tanh form, 0.044715
            u = (2 / _PI).sqrt() * (d + _dec.Decimal("0.044715") * d * d * d)
            a = -2 * u
            if a > 10 ** 5:
                return None
            return d / (1 + a.exp())
        if act == 2:                                  # GELU, erf form
            return _dec.Decimal("0.5") * d * dec_erfc(-d / _dec.Decimal(2).sqrt())
        if act == 3:                                  # SiLU
            if -d > 10 ** 5:
                return None
            return d / (1 + (-d).exp())
        return d if d > 0 else _dec.Decimal(0)       # ReLU


def round_grid(v: Fraction, mant: int, emin: int) -> Fraction:
    """Round a rational to nearest-even on the grid of a binary type with `mant`
    fraction bits and smallest normal exponent `emin` (subnormals included)."""
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    q = Fraction(2) ** (e - mant)
    return (1 if v > 0 else -1) * rne_int(a / q) * q
