"""Pins for the oracle's block-scaled GEMM (CPU only).

C[m,n] = bf16( sum_g P(m,n,g) * as[m,g] * ws[n/128,g] ),
P = sum_{k in group g} dec(aq[m,k]) * dec(wq[n,k]).
"""
from fractions import Fraction

import numpy as np
import pytest

import inputs
from tests import exact


def _e4m3_frac(code: int) -> Fraction:
    """Value of an e4m3fn code from its fields (format definition)."""
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    v = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if s else v


_E4 = [_e4m3_frac(c) if (c & 0x7F) != 0x7F else None for c in range(256)]


def _exact_gemm(aq, as_, wq, ws):
    M, K = aq.shape
    N = wq.shape[0]
    G = K // 128
    out = [[None] * N for _ in range(M)]
    mag = [[None] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            tot = Fraction(0)
            for g in range(G):
                P = sum(_E4[int(aq[m, k])] * _E4[int(wq[n, k])] for k in range(128 * g, 128 * g + 128))
                term = P * Fraction(float(as_[m, g])) * Fraction(float(ws[n // 128, g]))
                acc += term
                tot += abs(term)
            out[m][n] = acc
            mag[m][n] = tot
    return out, mag


def _bf16_bits_exact(v: Fraction, negative_zero=False) -> int:
    r = exact.rn_bf16(v)
    if r == 0:
        return 0x8000 if (v < 0 or negative_zero) else 0
    return exact.bf16_bits_of(r)


@pytest.mark.parametrize("M,K,N", [(1, 128, 128), (2, 256, 128), (1, 256, 256)])
def test_gemm_bruteforce_exact(ora, M, K, N):
    a = inputs.activations(21 + M, M, K, outliers=True)
    w = inputs.weights(22 + K, N, K)
    aq, as_ = ora.quant_act(a)
    wq, ws = ora.quant_weight(w)
    c, c64 = ora.gemm_block(aq, as_, wq, ws, want_f64=True)
    ex, mag = _exact_gemm(aq, as_, wq, ws)
    for m in range(M):
        for n in range(N):
            v = ex[m][n]
            # each group term takes two binary64 roundings and the sum one per group
            assert abs(Fraction(float(c64[m, n])) - v) <= mag[m][n] * Fraction(1, 2 ** 50), (m, n)
            # bitwise, unless the exact value sits within binary64 noise of a bf16 midpoint
            r = exact.rn_bf16(v)
            spacing_guard = mag[m][n] * Fraction(1, 2 ** 48)
            if abs(exact.rn_bf16(v + spacing_guard) - r) == 0 and abs(exact.rn_bf16(v - spacing_guard) - r) == 0:
                assert c[m, n] == _bf16_bits_exact(v), (m, n)


def _grid_values(r, shape):
    """Random e4m3 grid values (no NaN), as float32."""
    codes = r.integers(0, 256, shape).astype(np.uint8)
    codes = np.where((codes & 0x7F) == 0x7F, codes & 0xF0, codes)
    t = np.array([float(_E4[c]) if _E4[c] is not None else 0.0 for c in range(256)], np.float64)
    return t[codes].astype(np.float32), codes


def test_gemm_unit_scales_equals_plain_matmul(ora):
    """Values already on the e4m3 grid with every group's and block's max exactly
    448: quantisation is the identity with scale 1, so C is bf16 of the plain
    binary64 product A @ W^T (exact here: every product and partial sum fits)."""
    r = np.random.default_rng(31)
    M, K, N = 5, 384, 256
    A, _ = _grid_values(r, (M, K))
    W, _ = _grid_values(r, (N, K))
    A[:, ::128] = 448.0
    W[::128, ::128] = -448.0
    a = inputs.to_bf16_bits(A)
    w = inputs.to_bf16_bits(W)
    aq, as_ = ora.quant_act(a)
    wq, ws = ora.quant_weight(w)
    assert np.all(as_ == 1.0) and np.all(ws == 1.0)
    assert np.array_equal(ora.e4m3_table()[aq], A.astype(np.float64))
    ref = A.astype(np.float64) @ W.astype(np.float64).T
    c = ora.gemm_block(aq, as_, wq, ws)
    want = np.array([[_bf16_bits_exact(Fraction(float(v))) for v in row] for row in ref], np.uint16)
    assert np.array_equal(c, want)


@pytest.mark.parametrize("j", [-12, 0, 9])
def test_gemm_one_hot_row(ora, j):
    """A row with one non-zero value 448*2^j at column k0: its group gets code
    0x7E and scale 2^j, the others scale RN32(1e-10/448) and code 0, so
    C[n] = bf16(dec(wq[n,k0]) * ws[n/128, k0/128] * 448 * 2^j)."""
    K, N, k0 = 512, 256, 300
    A = np.zeros((1, K), np.float32)
    A[0, k0] = 448.0 * 2.0 ** j
    a = inputs.to_bf16_bits(A)
    w = inputs.weights(33, N, K)
    aq, as_ = ora.quant_act(a)
    wq, ws = ora.quant_weight(w)
    assert aq[0, k0] == 0x7E and as_[0, k0 // 128] == np.float32(2.0 ** j)
    c = ora.gemm_block(aq, as_, wq, ws)
    for n in range(N):
        v = _E4[int(wq[n, k0])] * Fraction(float(ws[n // 128, k0 // 128])) * 448 * Fraction(2) ** j
        assert c[0, n] == _bf16_bits_exact(v), n


def test_gemm_row_scale_covariance(ora):
    """Scaling a whole A row by 2^j scales its unrounded outputs by exactly 2^j."""
    a = inputs.activations(41, 3, 512)
    w = inputs.weights(42, 256, 512)
    wq, ws = ora.quant_weight(w)
    aq, as_ = ora.quant_act(a)
    _, c1 = ora.gemm_block(aq, as_, wq, ws, want_f64=True)
    a2 = inputs.to_bf16_bits(ora.bf16_value(a) * np.float32(8.0))
    aq2, as2 = ora.quant_act(a2)
    _, c2 = ora.gemm_block(aq2, as2, wq, ws, want_f64=True)
    assert np.array_equal(c2, 8.0 * c1)


def test_gemm_group_structure(ora):
    """Zeroing one K-group of W's codes removes exactly that group's term:
    C64 = C64(without group) + term, term = P * as * ws computed from the codes."""
    a = inputs.activations(43, 2, 384)
    w = inputs.weights(44, 128, 384)
    aq, as_ = ora.quant_act(a)
    wq, ws = ora.quant_weight(w)
    _, full = ora.gemm_block(aq, as_, wq, ws, want_f64=True)
    wq0 = wq.copy()
    wq0[:, 128:256] = 0
    _, part = ora.gemm_block(aq, as_, wq0, ws, want_f64=True)
    t = ora.e4m3_table()
    P = t[aq[:, 128:256]] @ t[wq[:, 128:256]].T
    term = P * as_[:, 1:2].astype(np.float64) * ws[0, 1].astype(np.float64)
    np.testing.assert_allclose(full - part, term, rtol=1e-12, atol=0)


def test_gemm_sampled_matches_full_and_threads(ora, monkeypatch):
    a = inputs.activations(51, 7, 640)
    w = inputs.weights(52, 384, 640)
    aq, as_ = ora.quant_act(a)
    wq, ws = ora.quant_weight(w)
    c, c64 = ora.gemm_block(aq, as_, wq, ws, want_f64=True)
    r = np.random.default_rng(3)
    ms = r.integers(0, 7, 50)
    ns = r.integers(0, 384, 50)
    cs, cs64 = ora.gemm_block_at(aq, as_, wq, ws, ms, ns, want_f64=True)
    assert np.array_equal(cs, c[ms, ns]) and np.array_equal(cs64, c64[ms, ns])
    monkeypatch.setattr(ora, "threads", lambda: 1)
    c1 = ora.gemm_block(aq, as_, wq, ws)
    assert np.array_equal(c1, c)


def test_tolerance_helper(ora):
    """The comparison rule: |g - o| <= 1e-2 RMS(o) + ulp_bf16(o)."""
    o = np.array([1.0, -2.0, 0.0, 1000.0])
    rms = np.sqrt(np.mean(o * o))
    g_ok = ora.bf16_round(o + np.array([0.01 * rms, 0, 0, 0]) * 0.99)
    ok, ratio, _ = ora.within_tolerance(g_ok, o)
    assert ok and ratio <= 1.0
    g_bad = ora.bf16_round(o + np.array([0, 0, 0.02 * rms, 0]))
    ok, ratio, _ = ora.within_tolerance(g_bad, o)
    assert not ok and ratio > 1.0
    assert ora.bf16_ulp(np.array([1.0]))[0] == 2.0 ** -7
    assert ora.bf16_ulp(np.array([0.0]))[0] == 2.0 ** -133
