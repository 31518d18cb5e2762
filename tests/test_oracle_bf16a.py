"""Pins for the oracle's bf16-activation variant (CPU only):
C[m][n] = bf16(sum_g ws[n/128][g] * sum_{k in g} a[m][k] * dec(wq[n][k])),
fp8 block weights against unquantised bf16 activations."""
from fractions import Fraction

import numpy as np
import pytest

import inputs
from tests import exact
from tests.test_oracle_gemm import _E4, _bf16_bits_exact, _grid_values


def _exact_bf16a(a_bits, wq, ws):
    M, K = a_bits.shape
    N = wq.shape[0]
    av = [[Fraction(float(v)) for v in row] for row in exact_bf16_values(a_bits)]
    out = [[None] * N for _ in range(M)]
    mag = [[None] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            tot = Fraction(0)
            for g in range(K // 128):
                P = sum(av[m][k] * _E4[int(wq[n, k])] for k in range(128 * g, 128 * g + 128))
                term = P * Fraction(float(ws[n // 128, g]))
                acc += term
                tot += sum(abs(av[m][k] * _E4[int(wq[n, k])]) for k in range(128 * g, 128 * g + 128)) \
                    * abs(Fraction(float(ws[n // 128, g])))
            out[m][n] = acc
            mag[m][n] = tot
    return out, mag


def exact_bf16_values(a_bits):
    return (a_bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("M,K,N", [(1, 128, 128), (2, 256, 128)])
def test_bf16a_bruteforce_exact(ora, M, K, N):
    a = inputs.activations(41 + M, M, K, outliers=True)
    wq, ws = ora.quant_weight(inputs.weights(42 + K, N, K))
    c, c64 = ora.gemm_block_bf16a(a, wq, ws, want_f64=True)
    ex, mag = _exact_bf16a(a, wq, ws)
    for m in range(M):
        for n in range(N):
            v = ex[m][n]
            assert abs(Fraction(float(c64[m, n])) - v) <= mag[m][n] * Fraction(1, 2 ** 45), (m, n)
            r = exact.rn_bf16(v)
            guard = mag[m][n] * Fraction(1, 2 ** 44)
            if exact.rn_bf16(v + guard) == r and exact.rn_bf16(v - guard) == r:
                assert c[m, n] == _bf16_bits_exact(v), (m, n)


def test_bf16a_unit_scales_equals_plain_matmul(ora):
    """Weights on the e4m3 grid with every block's max 448 (scale 1) and small-integer activations: every
    product and sum is exact in binary64, so C is bf16 of numpy's A @ W^T."""
    r = np.random.default_rng(51)
    M, K, N = 4, 384, 256
    W, _ = _grid_values(r, (N, K))
    W[::128, ::128] = 448.0
    wq, ws = ora.quant_weight(inputs.to_bf16_bits(W))
    assert np.all(ws == 1.0)
    A = r.integers(-20, 21, (M, K)).astype(np.float32)
    ref = A.astype(np.float64) @ W.astype(np.float64).T
    c = ora.gemm_block_bf16a(inputs.to_bf16_bits(A), wq, ws)
    assert np.array_equal(c, ora.bf16_round(ref))


def test_bf16a_equals_quantised_path_on_exact_groups(ora):
    """Activation groups already of the form (e4m3 value) * 2^j with max exactly 448 * 2^j quantise exactly
    (codes = the values / 2^j, scale 2^j), so the bf16-activation GEMM equals the block GEMM bit for bit."""
    r = np.random.default_rng(52)
    M, K, N = 3, 512, 256
    A, _ = _grid_values(r, (M, K))
    A[:, ::128] = 448.0
    j = r.integers(-6, 7, (M, K // 128)).astype(np.float64)
    A = (A.astype(np.float64) * np.repeat(2.0 ** j, 128, axis=1)).astype(np.float32)
    a = inputs.to_bf16_bits(A)
    wq, ws = ora.quant_weight(inputs.weights(53, N, K))
    aq, as_ = ora.quant_act(a)
    assert np.array_equal(as_, (2.0 ** j).astype(np.float32))
    assert np.array_equal(ora.gemm_block_bf16a(a, wq, ws), ora.gemm_block(aq, as_, wq, ws))


@pytest.mark.parametrize("v", [1.0, -0.3125, 3.0e5])
def test_bf16a_one_hot_row(ora, v):
    """A row with one non-zero value v at column k0: C[n] = bf16(v * dec(wq[n,k0]) * ws[n/128, k0/128])."""
    K, N, k0 = 512, 256, 200
    A = np.zeros((1, K), np.float32)
    A[0, k0] = v
    a = inputs.to_bf16_bits(A)
    wq, ws = ora.quant_weight(inputs.weights(54, N, K))
    c = ora.gemm_block_bf16a(a, wq, ws)
    av = Fraction(float(exact_bf16_values(a)[0, k0]))
    for n in range(N):
        want = av * _E4[int(wq[n, k0])] * Fraction(float(ws[n // 128, k0 // 128]))
        assert c[0, n] == _bf16_bits_exact(want), n


def test_bf16a_power_of_two_covariance(ora):
    """Scaling every activation by 2^j scales every output by exactly 2^j (no overflow or underflow)."""
    a = inputs.activations(55, 2, 256, outliers=True)
    wq, ws = ora.quant_weight(inputs.weights(56, 128, 256))
    c0 = ora.bf16_value(ora.gemm_block_bf16a(a, wq, ws)).astype(np.float64)
    for j in (-5, 3):
        a2 = inputs.to_bf16_bits(exact_bf16_values(a) * np.float32(2.0 ** j))
        c2 = ora.bf16_value(ora.gemm_block_bf16a(a2, wq, ws)).astype(np.float64)
        assert np.array_equal(c2, c0 * 2.0 ** j)
