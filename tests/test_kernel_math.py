"""Host-side checks of arithmetic identities the GPU kernels rely on (CPU only).

The quant kernels divide by the group scale with one reciprocal per group and
a fused multiply-add correction instead of a full division per element.  The
claim checked here, exhaustively over its whole domain, is that this gives the
same e4m3 code as the correctly rounded quotient: every bf16 amax (the eps
floor included) and every bf16 a with |a| <= amax, both signs.  The GPU
kernels themselves are checked against the oracle in the gpu tests.
"""
import pytest


@pytest.mark.slow
def test_division_correction_matches_correct_rounding(pins, ora):
    bad = pins.pin_div_correction_mismatches(0, 0x7F80, ora.threads())
    assert bad == 0


def test_scale_formula_matches_division(pins):
    """s = max(amax, 1e-10f) / 448 by multiply-and-correct equals the correctly
    rounded division for every bf16 amax."""
    assert pins.pin_scale_formula_mismatches() == 0
