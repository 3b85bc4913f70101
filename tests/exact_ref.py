"""Exact-arithmetic checkers used to pin the oracle (never used by the product path).

These are independent of the oracle's C arithmetic: they work on Python ``Fraction``s and on
brute-force nearest-value search, so a mistake in the oracle's encoder, its scale division or
its bf16 rounding cannot hide behind the same mistake here.
"""
from fractions import Fraction

import numpy as np
import torch


def e4m3_values_torch() -> np.ndarray:
    """Value of every code 0..255 as decoded by torch's float8_e4m3fn (a library routine)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


_POS_VALS = None


def _pos_table():
    """Sorted non-negative finite E4M3 values (codes 0x00..0x7E are already increasing)."""
    global _POS_VALS
    if _POS_VALS is None:
        v = e4m3_values_torch()[:0x7F]
        assert np.all(np.diff(v) > 0)
        _POS_VALS = v
    return _POS_VALS


def e4m3_nearest(x: float) -> int:
    """Nearest E4M3 code by search over the value table: ties go to the even code (code and
    mantissa share the lowest bit), |x| >= 448 saturates, the sign of zero is kept."""
    x = float(x)
    sign = 0x80 if np.signbit(x) else 0
    a = abs(x)
    vals = _pos_table()
    if a >= vals[-1]:
        return sign | 0x7E
    hi = int(np.searchsorted(vals, a, side="left"))
    if vals[hi] == a:
        return sign | hi
    lo = hi - 1
    fa = Fraction(a)
    dlo = fa - Fraction(float(vals[lo]))
    dhi = Fraction(float(vals[hi])) - fa
    if dlo < dhi:
        c = lo
    elif dhi < dlo:
        c = hi
    else:
        c = lo if lo % 2 == 0 else hi
    return sign | c


def round_to_binary(fr: Fraction, p: int, emin: int) -> Fraction:
    """Round a rational to the nearest value of a binary format with p significant bits and
    minimum normal exponent emin (gradual underflow), ties to even.  No overflow handling."""
    if fr == 0:
        return Fraction(0)
    neg = fr < 0
    a = -fr if neg else fr
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - p + 1)
    n = a / ulp
    r = n.numerator // n.denominator
    rem = n - r
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and r % 2 == 1):
        r += 1
    out = r * ulp
    return -out if neg else out


def rn32(fr: Fraction) -> Fraction:
    return round_to_binary(fr, 24, -126)


def rn_bf16(fr: Fraction) -> Fraction:
    return round_to_binary(fr, 8, -126)


def f32_of(fr: Fraction) -> np.float32:
    """A rational that is exactly a binary32 value, as np.float32 (asserts exactness)."""
    f = np.float32(float(fr))
    assert Fraction(float(f)) == fr, "value is not a binary32"
    return f


def bf16_bits_of(fr: Fraction, negative_zero: bool = False) -> int:
    """A rational that is exactly a bf16 value -> its bit pattern."""
    f = f32_of(fr)
    b = int(np.array([f], np.float32).view(np.uint32)[0]) >> 16
    if fr == 0 and negative_zero:
        b |= 0x8000
    return b
