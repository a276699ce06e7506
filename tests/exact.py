"""Exact-arithmetic helpers for pinning the oracle (rational numbers, no floats).

These re-derive roundings from first principles with ``fractions.Fraction`` so
that the oracle's numpy roundings are checked against something other than
themselves.
"""
from fractions import Fraction


def round_fraction(fr: Fraction, sig_bits: int, min_exp: int) -> Fraction:
    """Round an exact rational to a binary float grid, ties to even.

    ``sig_bits`` significant bits (including the implicit one); ``min_exp`` is
    the exponent of the smallest normal number (values below it use the fixed
    subnormal step 2**(min_exp - sig_bits + 1)).  No overflow handling.
    """
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    # exponent e with 2**e <= a < 2**(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, min_exp)
    step = Fraction(2) ** (e - sig_bits + 1)
    q = a / step
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * step


def to_f32(fr):
    return round_fraction(Fraction(fr), 24, -126)


def to_f16(fr):
    return round_fraction(Fraction(fr), 11, -14)


def to_bf16(fr):
    return round_fraction(Fraction(fr), 8, -126)


def round_half_even_int(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl
