"""Exact rational rounding (fractions.Fraction) for the op-order pins.

Test infrastructure: written from the IEEE 754 definition of round to
nearest, ties to even, independently of the oracle and of the GPU library.
The two readings of each formula are spelled out so that a test can check
which one a result follows. The case tables hold inputs (found by a search
for disagreements between the readings), not expected values.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np


def round_binary(fr: Fraction, frac_bits: int, min_exp: int) -> Fraction:
    """Round a rational to the nearest binary float with frac_bits fraction
    bits and normal exponents >= min_exp (ties to even; subnormals below)."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                                   # now 2^e <= a < 2^(e+1)
    lsb = Fraction(2) ** (max(e, min_exp) - frac_bits)
    q, rem = divmod(a, lsb)
    if rem * 2 > lsb or (rem * 2 == lsb and q % 2 == 1):
        q += 1
    return sign * q * lsb


def rn32(fr: Fraction) -> Fraction:
    return round_binary(fr, 23, -126)


def rn_bf16(fr: Fraction) -> Fraction:
    return round_binary(fr, 7, -126)


def rint_even(fr: Fraction) -> int:
    q, rem = divmod(fr, 1)
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and q % 2 == 1):
        q += 1
    return int(q)


def f32(fr: Fraction) -> np.float32:
    return np.float32(float(fr))


def quant_reciprocal(v: Fraction, amax: Fraction) -> int:
    """The reading taken: q = rint(RN32(v * RN32(127 / amax)))."""
    return rint_even(rn32(v * rn32(Fraction(127) / amax)))


def quant_divide(v: Fraction, amax: Fraction) -> int:
    """The other reading of round(Wr / s_w): q = rint(RN32(v / RN32(amax / 127)))."""
    return rint_even(rn32(v / rn32(amax / 127)))


# (v, amax) as float32 hex: a general pair, and pairs with v / amax = 1/2
# exactly (the exact code is the tie 63.5; each reading's rounding of the
# reciprocal or of the scale pushes it a different way)
QUANT_ORDER_CASES = [
    ("-0x1.95814ap+5", "0x1.bfd192p+6"),
    ("0x1.bbed66p-17", "0x1.d7c9f6p-17"),
    ("0x1.3p+11", "0x1.3p+12"),
    ("0x1.8ep+1", "0x1.8ep+2"),
    ("0x1.64p+17", "0x1.64p+18"),
    ("0x1.5ep-21", "0x1.5ep-20"),
]


# (acc, s_w, s_x): the two fp32 products land on either side of a bf16
# rounding boundary
EPILOGUE_ORDER_CASES = [
    (451142, "0x1.88e50ep-9", "0x1.2e212ep-11"),
    (-85083, "0x1.f3b3f6p-12", "0x1.883d5ep-8"),
    (-319191, "0x1.d65c4p-9", "0x1.b5283p-12"),
    (549653, "0x1.1a8ceep-13", "0x1.4aff36p-12"),
    (884965, "0x1.9161ep-9", "0x1.822b0ap-8"),
]


def epilogue_weight_first(acc: int, sw: Fraction, sx: Fraction) -> Fraction:
    """The reading taken: RN_bf16(RN32(RN32(acc * s_w) * s_x[m]))."""
    return rn_bf16(rn32(rn32(rn32(Fraction(acc)) * sw) * sx))


def epilogue_scales_first(acc: int, sw: Fraction, sx: Fraction) -> Fraction:
    """The other order: RN_bf16(RN32(acc * RN32(s_w * s_x[m])))."""
    return rn_bf16(rn32(rn32(Fraction(acc)) * rn32(sw * sx)))
