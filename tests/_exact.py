"""Exact rational arithmetic with IEEE binary32 round-to-nearest-even.

Used to check, by brute force on small inputs, that the oracle rounds each
operation exactly once: every value is carried as a Fraction and rounded to
fp32 explicitly after each operation.  Independent of numpy/libm rounding.
"""
from fractions import Fraction
from math import isqrt

import numpy as np

_TWO = Fraction(2)
_MAX_EXP = 127
_MIN_NORMAL_EXP = -126
_MANT = 23


def exact(x) -> Fraction:
    """Exact value of a finite float (fp32 or fp64)."""
    return Fraction(float(x))


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if _TWO ** e > a:
        e -= 1
    elif _TWO ** (e + 1) <= a:
        e += 1
    return e


def rne_f32(q: Fraction, sticky: bool = False) -> np.float32:
    """Round q (plus an infinitesimal positive amount when `sticky`) to fp32."""
    if q == 0:
        return np.float32(0.0)
    neg = q < 0
    a = -q if neg else q
    e = _floor_log2(a)
    qexp = max(e, _MIN_NORMAL_EXP) - _MANT          # exponent of one unit in the last place
    scaled = a / _TWO ** qexp
    n = scaled.numerator // scaled.denominator
    r = scaled - n
    half = Fraction(1, 2)
    if r > half or (r == half and (sticky or n % 2 == 1)):
        n += 1
    val = Fraction(n) * _TWO ** qexp
    if val >= _TWO ** (_MAX_EXP + 1):
        out = np.float32(np.inf)
    else:
        out = np.float32(float(val))                  # exact: val is an fp32 value
    return -out if neg else out


def sqrt_rne_f32(x: Fraction) -> np.float32:
    """Correctly rounded fp32 square root of a non-negative dyadic rational."""
    if x < 0:
        raise ValueError
    if x == 0:
        return np.float32(0.0)
    num, den = x.numerator, x.denominator               # den = 2^k (x is dyadic)
    k = den.bit_length() - 1
    s = max(200, (k + 400) // 2)                        # extra bits: far beyond fp32's 24
    shift = 2 * s - k                                   # sqrt(x) * 2^s = sqrt(num << shift)
    assert shift >= 0 and den == 1 << k
    big = num << shift
    r = isqrt(big)
    s_eff = Fraction(1, 2 ** s)
    exact_root = r * r == big
    return rne_f32(Fraction(r) * s_eff, sticky=not exact_root)


def f32(x) -> np.float32:
    return np.float32(x)


# exact operations, each rounded once
def add(a, b):
    return rne_f32(exact(a) + exact(b))


def sub(a, b):
    return rne_f32(exact(a) - exact(b))


def mul(a, b):
    return rne_f32(exact(a) * exact(b))


def div(a, b):
    return rne_f32(exact(a) / exact(b))


def sqrt(a):
    return sqrt_rne_f32(exact(a))
