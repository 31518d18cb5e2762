"""Exact rational rounding, used to pin the oracle by brute force.

Every helper takes a ``fractions.Fraction`` and returns the exactly rounded
value as a Fraction, following only the definition of a binary floating-point
format: p significant bits, smallest normal exponent emin, subnormal spacing
2^(emin - p + 1), round to nearest with ties to the even significand.
"""
from fractions import Fraction

import numpy as np


def _floor_log2(x: Fraction) -> int:
    # exact floor(log2(x)) for x > 0
    n, d = x.numerator, x.denominator
    e = n.bit_length() - d.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    elif Fraction(2) ** (e + 1) <= x:
        e += 1
    return e


def round_binary(x: Fraction, p: int, emin: int) -> Fraction:
    """Round x to a binary float with p significant bits, min normal exponent emin
    (no overflow handling: the callers stay in range)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    ax = abs(x)
    e = max(_floor_log2(ax), emin)
    spacing = Fraction(2) ** (e - p + 1)
    q = ax / spacing
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * spacing


def rn_f32(x: Fraction) -> Fraction:
    return round_binary(x, 24, -126)


def rn_bf16(x: Fraction) -> Fraction:
    return round_binary(x, 8, -126)


E4M3_MAX = Fraction(448)


def rn_e4m3_sat(x: Fraction) -> Fraction:
    """Nearest e4m3fn value (4 significant bits, emin -6) with saturation at +-448."""
    r = round_binary(x, 4, -6)
    if abs(r) > E4M3_MAX:
        r = E4M3_MAX if r > 0 else -E4M3_MAX
    return r


def e4m3_code_of(v: Fraction, negative_zero: bool = False) -> int:
    """The code of an e4m3 grid value, from the format's field layout."""
    if v == 0:
        return 0x80 if negative_zero else 0x00
    sign = 0x80 if v < 0 else 0
    av = abs(v)
    if av < Fraction(1, 64):
        m = av / Fraction(1, 512)
        assert m.denominator == 1
        return sign | int(m)
    e = _floor_log2(av)
    m = (av / Fraction(2) ** e - 1) * 8
    assert m.denominator == 1 and 0 <= m < 8
    return sign | ((e + 7) << 3) | int(m)


def bf16_bits_of(v: Fraction) -> int:
    """Bits of a bf16 grid value (finite, representable)."""
    f = np.float32(float(v))
    assert Fraction(float(f)) == v
    return int(np.array([f], np.float32).view(np.uint32)[0] >> 16)


def frac_bf16(bits: int) -> Fraction:
    return Fraction(float(np.array([bits << 16], np.uint32).view(np.float32)[0]))


def frac_f32(x) -> Fraction:
    return Fraction(float(np.float32(x)))


EPS_F32 = frac_f32(np.float32(1e-10))


def quant_group_exact(bits):
    """Group quant by exact rationals: s = RN32(max(amax, eps) / 448),
    code = e4m3(RN32(a / s)).  Returns (codes, scale as Fraction)."""
    vals = [frac_bf16(int(b)) for b in bits]
    amax = max(abs(v) for v in vals)
    s = rn_f32(max(amax, EPS_F32) / 448)
    codes = []
    for b, v in zip(bits, vals):
        q = rn_e4m3_sat(rn_f32(v / s))
        neg = (int(b) & 0x8000) != 0
        codes.append(e4m3_code_of(q, negative_zero=neg))
    return codes, s
