"""Pins for the oracle's group quantisation (activation groups of 128 along K,
weight blocks of 128x128).  CPU only.

Rule under test (the workload's stated rule; the release pages name only the
per-token-group-128 quant): s = RN32(max(amax, 1e-10f) / 448), q = e4m3(RN32(a / s)).
"""
from fractions import Fraction

import numpy as np
import pytest

import inputs
from tests import exact


def _f32bits(x):
    return int(np.array([x], np.float32).view(np.uint32)[0])


def _random_rows(seed, M, K):
    r = np.random.default_rng(seed)
    z = r.standard_normal((M, K)).astype(np.float32)
    z *= np.exp2(r.integers(-20, 20, (M, 1))).astype(np.float32)   # per-row magnitudes
    return inputs.to_bf16_bits(z)


def _near_tie_rows(seed, n_groups):
    """Groups whose quotients a/s land near e4m3 rounding midpoints: for a random
    amax, the bf16 values closest to midpoint * s (and their neighbours)."""
    r = np.random.default_rng(seed)
    grid = []
    for c in range(0x7F):
        e, m = (c >> 3) & 15, c & 7
        grid.append(m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10))
    grid = np.array(grid)
    mids = (grid[:-1] + grid[1:]) / 2
    rows = []
    for _ in range(n_groups):
        amax = np.float32(np.exp2(r.uniform(-30, 30)))
        amax_b = inputs.to_bf16_bits(np.array([amax]))[0]
        s = float(exact.rn_f32(exact.frac_bf16(int(amax_b)) / 448))
        pick = r.choice(mids, 63)
        targets = (pick * s).astype(np.float32)
        tb = inputs.to_bf16_bits(targets).astype(np.int32)
        cand = np.concatenate([tb, tb + 1, tb - 1])[:126]
        cand = np.clip(cand, 0, int(amax_b)).astype(np.uint16)
        sign = (r.integers(0, 2, cand.size) << 15).astype(np.uint16)
        g = np.concatenate([[amax_b], cand | sign, [amax_b ^ 0x8000]]).astype(np.uint16)
        rows.append(g)
    return np.concatenate(rows)[None, :]


def _check_exact(ora, a_bits):
    q, s = ora.quant_act(a_bits)
    M, K = a_bits.shape
    for m in range(M):
        for g in range(K // 128):
            codes, sc = exact.quant_group_exact(a_bits[m, 128 * g:128 * g + 128])
            assert Fraction(float(s[m, g])) == sc, (m, g)
            assert q[m, 128 * g:128 * g + 128].tolist() == codes, (m, g)


def test_quant_act_exact_random(ora):
    _check_exact(ora, _random_rows(1, 3, 512))


def test_quant_act_exact_near_ties(ora):
    _check_exact(ora, _near_tie_rows(2, 40))


def test_quant_act_exact_edge_groups(ora):
    _check_exact(ora, inputs.quant_edge_groups())


def test_quant_act_invariants(ora):
    a = np.concatenate([_random_rows(3, 64, 1024), ], axis=0)
    q, s = ora.quant_act(a)
    t = ora.e4m3_table()
    vals = ora.bf16_value(a).astype(np.float64)
    G = a.shape[1] // 128
    for m in range(a.shape[0]):
        for g in range(G):
            v = vals[m, 128 * g:128 * (g + 1)]
            c = q[m, 128 * g:128 * (g + 1)]
            amax = np.max(np.abs(v))
            # (i) the group's largest magnitude maps to +-448
            at = np.abs(v) == amax
            assert np.all((c[at] & 0x7F) == 0x7E)
            # (iii) never the NaN codes
            assert not np.any((c & 0x7F) == 0x7F)
            # (vi) dequantisation error within half an e4m3 ulp of a/s (+ the fp32 quotient rounding)
            ratio = v / float(s[m, g])
            e = np.floor(np.log2(np.maximum(np.abs(ratio), 2.0 ** -6)))
            half_ulp = np.ldexp(1.0, (e - 4).astype(np.int64))
            err = np.abs(t[c] - ratio)
            assert np.all(err <= half_ulp + np.abs(ratio) * 2.0 ** -23 + 1e-300)


def test_quant_act_zero_group_and_sign(ora):
    a = np.zeros((2, 256), np.uint16)
    a[1, :] = 0x8000                                          # -0.0
    q, s = ora.quant_act(a)
    # (ii) all-zero groups: codes +-0, scale RN32(RN32(1e-10)/448) = 0x2A7B5123
    assert np.all(q[0] == 0x00) and np.all(q[1] == 0x80)
    assert all(_f32bits(x) == 0x2A7B5123 for x in s.ravel())
    want = exact.rn_f32(exact.EPS_F32 / 448)
    assert Fraction(float(s[0, 0])) == want
    # (iv) sign symmetry: q(-a) = q(a) ^ 0x80, same scale
    b = _random_rows(4, 8, 512)
    q1, s1 = ora.quant_act(b)
    q2, s2 = ora.quant_act(b ^ np.uint16(0x8000))
    assert np.array_equal(q2, q1 ^ np.uint8(0x80)) and np.array_equal(s1, s2)


@pytest.mark.parametrize("j", [-7, -1, 1, 5])
def test_quant_act_scale_covariance(ora, j):
    """(v) multiplying a group by 2^j leaves the codes and multiplies the scale by 2^j."""
    r = np.random.default_rng(5)
    z = (r.standard_normal((4, 512)) * 3).astype(np.float32)
    z = np.where(np.abs(z) < 1e-3, np.float32(1e-3), z)       # keep everything normal after scaling
    a = inputs.to_bf16_bits(z)
    b = inputs.to_bf16_bits(ora.bf16_value(a) * np.float32(2.0 ** j))
    qa, sa = ora.quant_act(a)
    qb, sb = ora.quant_act(b)
    assert np.array_equal(qa, qb)
    assert np.array_equal(sb, sa * np.float32(2.0 ** j))


def test_quant_weight_exact(ora):
    w = inputs.weights(9, 256, 256)
    w[0, 3] = 0x4300                                          # 128.0 in one block
    w[128:256, 128:256] = 0                                   # one all-zero block
    q, s = ora.quant_weight(w)
    assert s.shape == (2, 2)
    for bn in range(2):
        for bk in range(2):
            blk = w[128 * bn:128 * (bn + 1), 128 * bk:128 * (bk + 1)].ravel()
            codes, sc = exact.quant_group_exact(blk)
            assert Fraction(float(s[bn, bk])) == sc
            assert q[128 * bn:128 * (bn + 1), 128 * bk:128 * (bk + 1)].ravel().tolist() == codes
    assert np.all((q[128:, 128:] & 0x7F) == 0)


def test_quant_weight_blocks_are_independent(ora):
    w = inputs.weights(10, 384, 256)
    q1, s1 = ora.quant_weight(w)
    w2 = w.copy()
    w2[130, 200] = 0x4700                                     # 32768.0 in block (1, 1)
    q2, s2 = ora.quant_weight(w2)
    changed = np.argwhere(s1 != s2).tolist()
    assert changed == [[1, 1]]
    mask = np.ones_like(q1, bool)
    mask[128:256, 128:256] = False
    assert np.array_equal(q1[mask], q2[mask])


def test_quant_act_thread_independent(ora, monkeypatch):
    a = _random_rows(11, 33, 640)
    q8, s8 = ora.quant_act(a)
    monkeypatch.setattr(ora, "threads", lambda: 1)
    q1, s1 = ora.quant_act(a)
    assert np.array_equal(q1, q8) and np.array_equal(s1, s8)
