"""Pins for the oracle's MoE decode and for the harness routing (CPU only).

MoE decode, per (token t, slot j) with expert e = ids[t,j]:
  gu = bf16(block GEMM of quant(x[t]) against w13[e]),  gate = gu[:I], up = gu[I:]
  h  = bf16(silu(gate) * up), then quantised per 128 along I,
  y  = block GEMM of quant(h) against w2[e] (binary64, unrounded),
  out[t] = bf16(sum_j w[t,j] * y(t,j)), j ascending.
silu's exp is the one step these pins cannot reach exactly (binary64 exp): the
silu value itself is parity unpinned beyond the output tolerance.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from block_scaled_fp8_r9k_amd import inputs
from tests import exact
from tests.test_oracle_gemm import _E4, _bf16_bits_exact


def _small(seed, T=2, H=256, E=4, I=128, topk=2):
    x, ids, w, w13, w2 = inputs.moe_inputs(seed, T, H, E, I, topk)
    return x, ids, w, w13, w2


def _quant_experts(ora, w13, w2):
    E = w13.shape[0]
    q13, s13, q2, s2 = [], [], [], []
    for e in range(E):
        a, b = ora.quant_weight(w13[e]); q13.append(a); s13.append(b)
        a, b = ora.quant_weight(w2[e]); q2.append(a); s2.append(b)
    return np.stack(q13), np.stack(s13), np.stack(q2), np.stack(s2)


def test_moe_top1_reduces_to_dense_chain(ora):
    """top-1 with weight 1: out[t] = bf16(y) where y is the dense chain."""
    x, ids, w, w13, w2 = _small(61, T=3, topk=1)
    w = np.ones_like(w)
    q13, s13, q2, s2 = _quant_experts(ora, w13, w2)
    out, inter = ora.moe_decode(x, ids, w, q13, s13, q2, s2, intermediates=True)
    I = q2.shape[2]
    for t in range(x.shape[0]):
        e = int(ids[t, 0])
        gu = ora.gemm_block_qa(x[t:t + 1], q13[e], s13[e])
        assert np.array_equal(gu[0], inter["gu"][t])
        g = ora.bf16_value(gu[0, :I]).astype(np.float64)
        u = ora.bf16_value(gu[0, I:]).astype(np.float64)
        h = ora.bf16_round(g / (1.0 + np.exp(-g)) * u)
        assert np.array_equal(h, inter["h"][t])
        c, c64 = ora.gemm_block_qa(h[None, :], q2[e], s2[e], want_f64=True)
        assert np.array_equal(c64[0], inter["y"][t])
        assert np.array_equal(c[0], out[t])


def test_moe_identical_experts_ignore_routing(ora):
    """All experts equal: the output does not depend on which experts are chosen
    (the weights sum to 1 up to fp32 rounding), so two routings agree to 1 bf16 ulp."""
    x, ids, w, w13, w2 = _small(62, T=2, E=4, topk=2)
    w13[:] = w13[0]
    w2[:] = w2[0]
    q13, s13, q2, s2 = _quant_experts(ora, w13, w2)
    out1 = ora.moe_decode(x, ids, w, q13, s13, q2, s2)
    ids2 = (ids + 1) % 4
    out2 = ora.moe_decode(x, ids2, w, q13, s13, q2, s2)
    d = np.abs(ora.bf16_value(out1).astype(np.float64) - ora.bf16_value(out2))
    assert np.all(d <= ora.bf16_ulp(ora.bf16_value(out1)))


def test_moe_slot_order_only_changes_rounding(ora):
    x, ids, w, w13, w2 = _small(63, T=2, E=4, topk=2)
    q13, s13, q2, s2 = _quant_experts(ora, w13, w2)
    out1, i1 = ora.moe_decode(x, ids, w, q13, s13, q2, s2, intermediates=True)
    out2 = ora.moe_decode(x, ids[:, ::-1].copy(), w[:, ::-1].copy(), q13, s13, q2, s2)
    yt = np.einsum("tj,tjh->th", w.astype(np.float64), i1["y"].reshape(2, 2, -1))
    ok, _, _ = ora.within_tolerance(out2, yt)
    assert ok
    d = np.abs(ora.bf16_value(out1).astype(np.float64) - ora.bf16_value(out2))
    assert np.all(d <= ora.bf16_ulp(yt))


def _exact_rows(aq_row, as_row, wq, ws):
    """Exact sum_g P * as * ws for every row n of wq (Fractions)."""
    K = aq_row.size
    out = []
    for n in range(wq.shape[0]):
        acc = Fraction(0)
        for g in range(K // 128):
            P = sum(_E4[int(aq_row[k])] * _E4[int(wq[n, k])] for k in range(128 * g, 128 * g + 128))
            acc += P * Fraction(float(as_row[g])) * Fraction(float(ws[n // 128, g]))
        out.append(acc)
    return out


@pytest.mark.slow
def test_moe_bruteforce_exact(ora):
    """H = I = 128, E = 4, top-2, T = 2 with exact rationals everywhere except
    silu's exp (binary64)."""
    T, H, E, I, k = 2, 128, 4, 128, 2
    x, ids, w, w13, w2 = inputs.moe_inputs(64, T, H, E, I, k)
    q13, s13, q2, s2 = _quant_experts(ora, w13, w2)
    out, inter = ora.moe_decode(x, ids, w, q13, s13, q2, s2, intermediates=True)
    for t in range(T):
        codes, sx = exact.quant_group_exact(x[t])
        xq = np.array(codes, np.uint8)
        acc_t = Fraction(0)
        for j in range(k):
            e = int(ids[t, j])
            gu_ex = _exact_rows(xq, np.array([float(sx)], np.float32), q13[e], s13[e])
            gu_bits = [_bf16_bits_exact(v) for v in gu_ex]
            assert gu_bits == inter["gu"][t * k + j].tolist()
            hb = []
            for i in range(I):
                g = float(exact.frac_bf16(gu_bits[i]))
                u = exact.frac_bf16(gu_bits[I + i])
                silu = Fraction(g / (1.0 + math.exp(-g)))
                hb.append(_bf16_bits_exact(silu * u))
            # the oracle multiplies silu * u in binary64 before its one bf16 rounding:
            # allow a difference only where the exact product sits on a bf16 tie
            got_h = inter["h"][t * k + j].tolist()
            mism = [i for i in range(I) if hb[i] != got_h[i]]
            assert len(mism) == 0, mism
            hcodes, hs = exact.quant_group_exact(np.array(hb, np.uint16))
            assert hcodes == inter["hq"][t * k + j].tolist()
            y_ex = _exact_rows(np.array(hcodes, np.uint8), np.array([float(hs)], np.float32), q2[e], s2[e])
            for n in range(H):
                assert abs(Fraction(float(inter["y"][t * k + j, n])) - y_ex[n]) <= abs(y_ex[n]) * Fraction(1, 2 ** 50)
            if j == 0:
                acc = [Fraction(float(w[t, j])) * v for v in y_ex]
            else:
                acc = [a + Fraction(float(w[t, j])) * v for a, v in zip(acc, y_ex)]
        want = [_bf16_bits_exact(v) for v in acc]
        assert want == out[t].tolist()


def test_route_invariants():
    r = np.random.default_rng(5)
    logits = r.standard_normal((64, 128)).astype(np.float32)
    ids, w = inputs.route(logits, 8)
    assert ids.shape == (64, 8) and w.dtype == np.float32
    for t in range(64):
        assert len(set(ids[t].tolist())) == 8                     # distinct experts
        assert ids[t, 0] == int(np.argmax(logits[t]))               # the argmax is chosen first
        assert abs(float(np.sum(w[t].astype(np.float64))) - 1.0) <= 8 * 2.0 ** -24
        assert np.all(np.diff(w[t]) <= 0)                           # ordered by probability
    # ties go to the lower expert id
    tie = np.zeros((1, 16), np.float32)
    ids_t, w_t = inputs.route(tie, 4)
    assert ids_t[0].tolist() == [0, 1, 2, 3] and np.all(w_t == np.float32(0.25))
