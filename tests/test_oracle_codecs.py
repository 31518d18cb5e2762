"""Pins for the oracle's e4m3fn and bf16 codecs (CPU only).

The e4m3fn format is the OCP 8-bit floating point E4M3 encoding (bias 7, no
infinities, S.1111.111 is NaN, largest finite 448); bf16 is the top half of an
IEEE binary32.  Each test checks the oracle against something other than its
own formula: closed-form values of the format, an integer bit-manipulation
encoder, a nearest-value search, or exact rationals.
"""
from fractions import Fraction

import numpy as np
import pytest

from tests import exact


def test_e4m3_closed_form_values(ora):
    # values fixed by the format definition
    assert ora.e4m3_value(0x7E) == 448.0
    assert ora.e4m3_value(0xFE) == -448.0
    assert ora.e4m3_value(0x08) == 2.0 ** -6       # smallest normal
    assert ora.e4m3_value(0x01) == 2.0 ** -9       # smallest subnormal
    assert ora.e4m3_value(0x07) == 7 * 2.0 ** -9   # largest subnormal
    assert ora.e4m3_value(0x38) == 1.0
    assert ora.e4m3_value(0x77) == 240.0
    assert ora.e4m3_value(0x00) == 0.0 and np.signbit(ora.e4m3_value(0x80))
    assert np.isnan(ora.e4m3_value(0x7F)) and np.isnan(ora.e4m3_value(0xFF))
    t = ora.e4m3_table()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must be strictly increasing"
    assert np.array_equal(t[0x80:0xFF], -pos)
    assert np.sum(np.isnan(t)) == 2


def test_e4m3_roundtrip_every_code(ora):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = ora.e4m3_table()[codes].astype(np.float32)
    assert np.array_equal(ora.e4m3_encode(vals), codes)


def test_e4m3_special_inputs(ora):
    x = np.array([np.inf, -np.inf, np.nan, 1e30, -1e30, 464.0, 470.0, 2.0 ** -10, -(2.0 ** -10),
                  2.0 ** -10 * (1 + 2 ** -20), 3 * 2.0 ** -10, 5 * 2.0 ** -10, -0.0, 0.0], np.float32)
    want = [0x7E, 0xFE, 0x7F, 0x7E, 0xFE, 0x7E, 0x7E, 0x00, 0x80, 0x01, 0x02, 0x02, 0x80, 0x00]
    assert ora.e4m3_encode(x).tolist() == want


def _exhaustive(ora, pins, fn_name, kind):
    import ctypes
    fn = ctypes.cast(getattr(ora.lib(), fn_name), ctypes.c_void_p).value
    first = ctypes.c_uint32(0)
    bad = pins.pin_exhaustive(fn, kind, ora.threads(), ctypes.byref(first))
    return bad, first.value


@pytest.mark.slow
def test_e4m3_exhaustive_against_bit_encoder(ora, pins):
    """Every binary32 pattern: the oracle (power-of-two scaling + rint) and the
    integer bit encoder agree."""
    bad, first = _exhaustive(ora, pins, "ora_e4m3_encode", 0)
    assert bad == 0, f"{bad} mismatches, first at pattern {first:#010x}"


def _near_grid_inputs():
    """Binary32 values within 8 ulps of every e4m3 value and every midpoint,
    both signs, plus random values over the whole exponent range."""
    t = []
    for c in range(0x7F):
        e, m = (c >> 3) & 15, c & 7
        t.append(m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10))
    t = np.array(t)
    centers = np.concatenate([t, (t[:-1] + t[1:]) / 2, [448.0 + 16.0, 2.0 ** -10]])
    c32 = centers.astype(np.float32).view(np.int32).astype(np.int64)
    offs = np.arange(-8, 9)
    pats = (c32[:, None] + offs[None, :]).ravel()
    pats = pats[(pats >= 0) & (pats < 0x7F800000)].astype(np.uint32)
    x = pats.view(np.float32)
    r = np.random.default_rng(1234)
    rnd = (r.integers(0, 0x7F800000, 2_000_000, dtype=np.int64)).astype(np.uint32).view(np.float32)
    x = np.concatenate([x, rnd])
    return np.concatenate([x, -x])


def test_e4m3_against_nearest_search(ora, pins):
    import ctypes
    x = np.ascontiguousarray(_near_grid_inputs())
    a = ora.e4m3_encode(x)
    b = np.empty(x.size, np.uint8)
    pins.pin_e4m3_encode_search_array(x.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), x.size,
                                      b.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), ora.threads())
    bad = np.nonzero(a != b)[0]
    assert bad.size == 0, f"first mismatch at {x[bad[0]]!r}: oracle {a[bad[0]]:#x} search {b[bad[0]]:#x}"


def test_e4m3_against_exact_rationals(ora):
    x = _near_grid_inputs()[::97][:5000]
    got = ora.e4m3_encode(x)
    for xi, gi in zip(x, got):
        v = exact.rn_e4m3_sat(Fraction(float(xi)))
        assert gi == exact.e4m3_code_of(v, negative_zero=bool(np.signbit(xi))), xi


@pytest.mark.slow
def test_bf16_exhaustive_against_integer_rounding(ora, pins):
    """Every non-NaN binary32 value, widened to binary64: the oracle's bf16
    rounding and the integer round-half-even of the low 16 bits agree."""
    bad, first = _exhaustive(ora, pins, "ora_bf16_round", 1)
    assert bad == 0, f"{bad} mismatches, first at pattern {first:#010x}"


def test_bf16_from_f64_rounds_once(ora):
    """A binary64 value just above a bf16 midpoint must round up; rounding
    through binary32 first would land on the midpoint and round to even."""
    x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8,
                  -(1.0 + 2.0 ** -8 + 2.0 ** -30), 2.0 ** -130 + 2.0 ** -140, 3.4e38, 1e-50], np.float64)
    got = ora.bf16_round(x)
    for xi, gi in zip(x, got):
        ax = abs(Fraction(xi))
        if ax >= Fraction(2) ** 128 - Fraction(2) ** 119:     # past the largest bf16 + half ulp
            want = 0x7F80 | (0x8000 if xi < 0 else 0)
        else:
            want = exact.bf16_bits_of(exact.rn_bf16(Fraction(xi))) if exact.rn_bf16(Fraction(xi)) != 0 else (
                0x8000 if xi < 0 else 0)
        assert gi == want, (xi, hex(gi), hex(want))
    assert got[0] == 0x3F81 and got[1] == 0x3F80 and got[2] == 0x3F82


def test_bf16_from_f64_random_against_exact(ora):
    r = np.random.default_rng(7)
    x = r.standard_normal(3000) * np.exp2(r.integers(-140, 120, 3000))
    got = ora.bf16_round(x)
    for xi, gi in zip(x, got):
        v = exact.rn_bf16(Fraction(float(xi)))
        want = exact.bf16_bits_of(v) if v != 0 else (0x8000 if xi < 0 else 0)
        assert gi == want, (xi, hex(gi), hex(want))
