"""Exact-rational model of the IEEE-754 operations the method uses (a pin).

Every binary32 value is exactly a Python float, so values travel as floats;
each operation is carried out exactly with ``fractions.Fraction`` and then
rounded to the target format by the textbook definition of
round-to-nearest-even: pick the quantum 2^q of the target format at the
value's binade (never below the subnormal quantum), and round the exact
quotient value / 2^q to the nearest integer, ties to the even one.

This shares nothing with the C oracle: no hardware float arithmetic decides a
result here, so a contracted multiply-add, a double rounding or a flushed
subnormal in the oracle shows up as a mismatch.
"""
from __future__ import annotations

import math
from fractions import Fraction

# (precision p incl. the hidden bit, minimum normal exponent, maximum exponent)
BINARY32 = (24, -126, 127)
BINARY16 = (11, -14, 15)
BFLOAT16 = (8, -126, 127)


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    return e


def round_rne(a: Fraction, fmt) -> Fraction:
    """Round a > 0 to the nearest value of `fmt`, ties to even; inf as None."""
    p, emin, emax = fmt
    assert a > 0
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - (p - 1))
    scaled = a / quantum
    n = scaled.numerator // scaled.denominator
    rest = scaled - n
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * quantum
    largest = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if r > largest:
        return None
    return r


def _signbit(x: float) -> bool:
    return math.copysign(1.0, x) < 0


def _to_float(r, negative: bool) -> float:
    if r is None:
        return -math.inf if negative else math.inf
    v = float(r)  # exact: r is a binary32 value
    return -v if negative else v


def mul32(a: float, b: float) -> float:
    """fl32(a * b) for binary32 a, b (infinities allowed, NaN not)."""
    negative = _signbit(a) != _signbit(b)
    if math.isinf(a) or math.isinf(b):
        if a == 0 or b == 0:
            return math.nan
        return -math.inf if negative else math.inf
    exact = Fraction(a) * Fraction(b)
    if exact == 0:
        return -0.0 if negative else 0.0
    return _to_float(round_rne(abs(exact), BINARY32), exact < 0)


def add32(a: float, b: float) -> float:
    """fl32(a + b) for finite binary32 a, b."""
    exact = Fraction(a) + Fraction(b)
    if exact == 0:
        # an exact zero sum is +0 under round-to-nearest, unless both addends are -0
        return -0.0 if (_signbit(a) and _signbit(b) and a == 0 and b == 0) else 0.0
    return _to_float(round_rne(abs(exact), BINARY32), exact < 0)


def _encode_narrow(x: float, fmt, frac_bits: int, exp_bias: int) -> int:
    sign = 0x8000 if _signbit(x) else 0
    if x == 0:
        return sign
    if math.isinf(x):
        return sign | (((1 << (15 - frac_bits)) - 1) << frac_bits)
    r = round_rne(abs(Fraction(x)), fmt)
    if r is None:
        return sign | (((1 << (15 - frac_bits)) - 1) << frac_bits)
    if r == 0:  # below half the smallest subnormal: a signed zero
        return sign
    p, emin, _ = fmt
    e = _floor_log2(r)
    if e < emin:  # subnormal: integer multiple of the subnormal quantum
        q = r / Fraction(2) ** (emin - frac_bits)
        assert q.denominator == 1
        return sign | int(q)
    frac = r / Fraction(2) ** (e - frac_bits) - (1 << frac_bits)
    assert frac.denominator == 1 and 0 <= frac < (1 << frac_bits)
    return sign | ((e + exp_bias) << frac_bits) | int(frac)


def f16_bits(x: float) -> int:
    """IEEE binary16 encoding of x rounded to nearest even (x a finite binary32)."""
    return _encode_narrow(x, BINARY16, 10, 15)


def bf16_bits(x: float) -> int:
    """bfloat16 encoding of x rounded to nearest even (x a finite binary32)."""
    return _encode_narrow(x, BFLOAT16, 7, 127)


def nested_scale(scale_codebook_value: float, absmax: float, offset: float) -> float:
    """Scale of one block: fl32(fl32(codebook[code] * absmax) + offset)."""
    return add32(mul32(scale_codebook_value, absmax), offset)


def value(code_value: float, scale: float, out_dtype: str):
    """One output element in its stored form: float (F32) or uint16 bits."""
    v = mul32(code_value, scale)
    if out_dtype == "f32":
        return v
    if out_dtype == "f16":
        return f16_bits(v)
    if out_dtype == "bf16":
        return bf16_bits(v)
    raise ValueError(out_dtype)
