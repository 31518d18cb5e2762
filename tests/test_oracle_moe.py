"""Pins for the oracle's MoE decode, routing and routed sum (CPU only).

MoE decode, per (token t, slot j) with expert e = ids[t,j]:
  gu = bf16(block GEMM of quant(x[t]) against w13[e]),  gate = gu[:I], up = gu[I:]
  h  = bf16(silu(gate) * up), then quantised per 128 along I,
  y  = block GEMM of quant(h) against w2[e] (binary64, unrounded),
  out[t] = bf16(sum_j w[t,j] * y(t,j)), j ascending.
silu uses binary64 exp, which no pin reproduces bit for bit; instead silu is
pinned through the oracle's own stage entry point (ora_moe_silu_mul) by facts
that do not restate its formula: its zero and its slope 1/2 at zero, its two
limits, the identity silu(z) - silu(-z) = z on every bf16 z, the closed form
silu(ln 3) = (3/4) ln 3 and its minimum -W(1/e) (W the Lambert function).
The stage entry points themselves (silu*up, and the down stage from given h)
are pinned bit for bit against the whole chain.  A slot with an id outside
[0, E) contributes nothing.

Routing: the top-k logits (a larger logit first, ties to the lower id), with
weights exp(l_j - l_0) / sum_i exp(l_i - l_0) over the chosen slots.  The
routed sum with the shared expert: out[t] = bf16(sum_j w y + g s).
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import inputs
from tests import exact
from tests.test_oracle_gemm import _E4, _bf16_bits_exact


def _routed(seed, T, H, E, I, topk):
    import oracle
    oracle.build(force=False)
    x, logits, w13, w2 = inputs.moe_inputs(seed, T, H, E, I)
    ids, w = oracle.moe_route(logits, topk)
    return x, ids, w, w13, w2


def _small(seed, T=2, H=256, E=4, I=128, topk=2):
    return _routed(seed, T, H, E, I, topk)


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
    x, ids, w, w13, w2 = _routed(64, T, H, E, I, k)
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


def test_route_invariants(ora):
    r = np.random.default_rng(5)
    logits = r.standard_normal((64, 128)).astype(np.float32)
    ids, w = ora.moe_route(logits, 8)
    assert ids.shape == (64, 8) and w.dtype == np.float32
    for t in range(64):
        assert len(set(ids[t].tolist())) == 8                     # distinct experts
        assert ids[t, 0] == int(np.argmax(logits[t]))               # the argmax is chosen first
        assert abs(float(np.sum(w[t].astype(np.float64))) - 1.0) <= 8 * 2.0 ** -24
        assert np.all(np.diff(w[t]) <= 0)                           # ordered by probability
        # the chosen logits are the 8 largest: nothing left out is larger than the smallest chosen
        rest = np.delete(logits[t], ids[t])
        assert np.all(rest <= logits[t, ids[t, -1]])
    # ties go to the lower expert id
    tie = np.zeros((1, 16), np.float32)
    ids_t, w_t = ora.moe_route(tie, 4)
    assert ids_t[0].tolist() == [0, 1, 2, 3] and np.all(w_t == np.float32(0.25))
    # ties between some experts only: lower ids first among equals, larger logits before them
    lt = np.array([[0.5, 2.0, 0.5, 2.0, -1.0, 0.5]], np.float32)
    assert ora.moe_route(lt, 4)[0][0].tolist() == [1, 3, 0, 2]


def test_route_worked_example(ora):
    """Logits (0, ln 3): the weights of a top-2 are 1/4 and 3/4, the larger first."""
    lt = np.array([[0.0, math.log(3.0), -5.0]], np.float32)
    ids, w = ora.moe_route(lt, 2)
    assert ids[0].tolist() == [1, 0]
    l0, l1 = float(lt[0, 1]), float(lt[0, 0])
    e = math.exp(l1 - l0)
    assert w[0].tolist() == [np.float32(1.0 / (1.0 + e)), np.float32(e / (1.0 + e))]
    assert abs(float(w[0, 0]) - 0.75) < 1e-7 and abs(float(w[0, 1]) - 0.25) < 1e-7
    # top-1: the single weight is exactly 1
    ids1, w1 = ora.moe_route(np.random.default_rng(1).standard_normal((9, 33)).astype(np.float32), 1)
    assert np.all(w1 == np.float32(1.0))


def test_route_all_experts_is_the_softmax(ora):
    """topk = E: the weights are the softmax of the logits, in descending order (scipy's softmax)."""
    from scipy.special import softmax
    lt = np.random.default_rng(2).standard_normal((12, 24)).astype(np.float32)
    ids, w = ora.moe_route(lt, 24)
    p = softmax(lt.astype(np.float64), axis=1)
    for t in range(12):
        assert sorted(ids[t].tolist()) == list(range(24))
        np.testing.assert_allclose(w[t].astype(np.float64), p[t, ids[t]], rtol=2e-7, atol=0)


def test_route_shift_invariance(ora):
    """Adding a constant to every logit of a token changes neither the experts nor (beyond rounding) the weights."""
    # logits on a 2^-10 grid below 8 in magnitude, so that adding 0.5 is exact in fp32
    z = np.random.default_rng(3).standard_normal((20, 64))
    lt = (np.round(np.clip(z, -7, 7) * 1024) / 1024).astype(np.float32)
    ids, w = ora.moe_route(lt, 8)
    ids2, w2 = ora.moe_route(lt + np.float32(0.5), 8)
    assert np.array_equal(ids, ids2)
    np.testing.assert_allclose(w2, w, rtol=4e-7, atol=0)


def test_fold_reduces_to_the_routed_sum(ora):
    """No shared expert: the routed sum of ora_moe_decode's own y is its output, bit for bit."""
    T, H, E, I, k = 3, 256, 4, 128, 2
    x, ids, w, w13, w2 = _routed(7, T, H, E, I, k)
    q13, s13, q2, s2 = _quant_experts(ora, w13, w2)
    out, inter = ora.moe_decode(x, ids, w, q13, s13, q2, s2, intermediates=True)
    assert np.array_equal(ora.moe_fold(inter["y"], ids, w, E), out)


def test_fold_shared_term_closed_forms(ora):
    """y = 0: out = bf16(g * s); g = 1 by default; an out-of-range id adds nothing."""
    T, H, k, E = 4, 128, 3, 8
    r = np.random.default_rng(4)
    ids = r.integers(0, E, (T, k)).astype(np.int32)
    w = r.random((T, k)).astype(np.float32)
    s = inputs.to_bf16_bits(r.standard_normal((T, H)).astype(np.float32))
    g = r.random(T).astype(np.float32)
    y0 = np.zeros((T * k, H))
    sv = ora.bf16_value(s).astype(np.float64)
    assert np.array_equal(ora.moe_fold(y0, ids, w, E, shared=s), s)
    want = ora.bf16_round(sv * g[:, None].astype(np.float64))
    assert np.array_equal(ora.moe_fold(y0, ids, w, E, shared=s, shared_w=g), want)
    # one slot out of range: the same as its weight set to zero
    y = r.standard_normal((T * k, H))
    ids_bad = ids.copy(); ids_bad[1, 2] = E
    w_zero = w.copy(); w_zero[1, 2] = 0.0
    assert np.array_equal(ora.moe_fold(y, ids_bad, w, E, shared=s, shared_w=g),
                          ora.moe_fold(y, ids, w_zero, E, shared=s, shared_w=g))
    # the routed part plus the shared part, rounded once, against an independent fp64 sum
    ref = (np.einsum("tj,tjh->th", w.astype(np.float64), y.reshape(T, k, H)) + g[:, None] * sv)
    assert np.array_equal(ora.moe_fold(y, ids, w, E, shared=s, shared_w=g), ora.bf16_round(ref))


# ---- the oracle's stage entry points (the references of the GPU test's stages) ----

def test_silu_mul_stage_equals_the_chain(ora):
    """ora_moe_silu_mul on the chain's own gu rows gives the chain's h bit for bit, so the GPU test's
    stage-2 reference is the same function the whole-chain oracle applies."""
    for seed, (T, H, E, I, topk) in ((81, (3, 256, 4, 256, 2)), (82, (5, 512, 3, 384, 3)),
                                     (83, (16, 2048, 128, 768, 8))):
        x, ids, w, w13, w2 = _routed(seed, T, H, E, I, topk)
        used = np.unique(ids)
        if E > 8:  # the workload shape: quantise only the experts the routing touches
            q = {int(e): (ora.quant_weight(w13[e]), ora.quant_weight(w2[e])) for e in used}
            z13, z2 = np.zeros((2 * I, H), np.uint8), np.zeros((H, I), np.uint8)
            o13, o2 = np.zeros((2 * I // 128, H // 128), np.float32), np.zeros((H // 128, I // 128), np.float32)
            q13 = np.stack([q[e][0][0] if e in q else z13 for e in range(E)])
            s13 = np.stack([q[e][0][1] if e in q else o13 for e in range(E)])
            q2 = np.stack([q[e][1][0] if e in q else z2 for e in range(E)])
            s2 = np.stack([q[e][1][1] if e in q else o2 for e in range(E)])
        else:
            q13, s13, q2, s2 = _quant_experts(ora, w13, w2)
        out, inter = ora.moe_decode(x, ids, w, q13, s13, q2, s2, intermediates=True)
        assert np.array_equal(ora.moe_silu_mul(inter["gu"]), inter["h"])
        # the down stage from those h rows reproduces every later intermediate and the output
        out_h, inter_h = ora.moe_down_from_h(inter["h"], ids, w, q2, s2, intermediates=True)
        assert np.array_equal(inter_h["hq"], inter["hq"])
        assert np.array_equal(inter_h["hs"].view(np.uint32), inter["hs"].view(np.uint32))
        assert np.array_equal(inter_h["y"].view(np.uint64), inter["y"].view(np.uint64))
        assert np.array_equal(out_h, out)


def test_down_from_h_on_foreign_rows(ora):
    """moe_down_from_h on h rows that no gate_up produced (seeded bf16 rows): the quant of each row is the
    dense activation quant, each y is the dense exact GEMM of that row, and the output is the routed sum;
    out-of-range ids contribute nothing."""
    T, H, E, I, topk = 3, 256, 4, 256, 2
    x, ids, w, w13, w2 = _routed(84, T, H, E, I, topk)
    _, _, q2, s2 = _quant_experts(ora, w13, w2)
    h = inputs.activations(85, T * topk, I, outliers=True)
    ids = ids.copy()
    ids[1, 1] = E + 3                        # out of range: contributes nothing
    out, inter = ora.moe_down_from_h(h, ids, w, q2, s2, intermediates=True)
    hq, hs = ora.quant_act(h)
    for p in range(T * topk):
        t, j = divmod(p, topk)
        if ids[t, j] >= E:
            continue
        assert np.array_equal(inter["hq"][p], hq[p])
        assert np.array_equal(inter["hs"][p].view(np.uint32), hs[p].view(np.uint32))
        _, y64 = ora.gemm_block(hq[p:p + 1], hs[p:p + 1], q2[ids[t, j]], s2[ids[t, j]], want_f64=True)
        assert np.array_equal(inter["y"][p], y64[0])
    for t in range(T):
        acc = np.zeros(H, np.float64)
        for j in range(topk):
            if 0 <= ids[t, j] < E:
                acc += np.float64(w[t, j]) * inter["y"][t * topk + j]
        assert np.array_equal(out[t], ora.bf16_round(acc))


def _silu_bf16(ora, z_bits, u_bits=None):
    """h = bf16(silu(g) * u) through ora_moe_silu_mul, gate g = z (bf16 bits), up u (default 1.0)."""
    z_bits = np.asarray(z_bits, np.uint16).ravel()
    n = z_bits.size
    u_bits = np.full(n, 0x3F80, np.uint16) if u_bits is None else np.asarray(u_bits, np.uint16).ravel()
    # one pair per value: I = 128 columns, value i at gate column i % 128 of pair i // 128
    P = -(-n // 128)
    gate = np.zeros(P * 128, np.uint16)
    up = np.full(P * 128, 0x3F80, np.uint16)
    gate[:n] = z_bits
    up[:n] = u_bits
    gu = np.concatenate([gate.reshape(P, 128), up.reshape(P, 128)], axis=1)
    return ora.moe_silu_mul(gu).reshape(-1)[:n]


def _bits(ora, v):
    return inputs.to_bf16_bits(np.asarray(v, np.float32))


def test_silu_zero_and_slope_at_zero(ora):
    """silu(+-0) = 0, and silu(z) = z/2 to within z^2/4 near zero (the logistic function is 1/2 at 0):
    for z = 2^-j, j >= 10, the bf16 result is exactly 2^-(j+1)."""
    h = _silu_bf16(ora, np.array([0x0000, 0x8000], np.uint16))
    assert np.all(ora.bf16_value(h) == 0.0)
    for j in range(10, 40):
        z = _bits(ora, [2.0 ** -j, -(2.0 ** -j)])
        got = ora.bf16_value(_silu_bf16(ora, z)).astype(np.float64)
        assert got[0] == 2.0 ** -(j + 1) and got[1] == -(2.0 ** -(j + 1)), (j, got)


def test_silu_limits(ora):
    """Large |z|: silu(z) -> z (exactly, after bf16 rounding, from z = 16 on), and silu(-z) -> -z e^-z
    (the asymptote, whose relative error e^-z is far below a bf16 ulp).  A mirrored definition
    z / (1 + e^z) would swap the two limits."""
    for z in (16.0, 20.0, 24.0, 32.0, 40.0, 64.0):
        zb = _bits(ora, [z, -z])
        got = ora.bf16_value(_silu_bf16(ora, zb)).astype(np.float64)
        assert got[0] == z
        asym = -z * math.exp(-z)
        assert abs(got[1] - asym) <= ora.bf16_ulp(np.array([asym]))[0], (z, got[1], asym)


def test_silu_odd_part_identity(ora):
    """silu(z) - silu(-z) = z for every z (the logistic function satisfies s(z) + s(-z) = 1): checked on
    every finite bf16 z in [-64, 64], to the two bf16 roundings."""
    allb = np.arange(0x0000, 0x8000, dtype=np.uint16)
    v = ora.bf16_value(allb).astype(np.float64)
    zb = allb[(v > 0) & (v <= 64)]
    z = ora.bf16_value(zb).astype(np.float64)
    hp = ora.bf16_value(_silu_bf16(ora, zb)).astype(np.float64)
    hn = ora.bf16_value(_silu_bf16(ora, zb | np.uint16(0x8000))).astype(np.float64)
    slack = 0.5 * ora.bf16_ulp(hp) + 0.5 * ora.bf16_ulp(np.abs(hn) + 1e-300)
    assert np.all(np.abs(hp - hn - z) <= slack * (1 + 1e-12))


def test_silu_closed_forms(ora):
    """silu(ln 3) = (3/4) ln 3 (the logistic function is 3/4 there), up to the bf16 rounding of ln 3 (the
    slope of silu near ln 3 is below 1.1) and of the result; and silu's minimum, -W(1/e) = -0.27846...
    at z = -1 - W(1/e) (W the Lambert function), matches the smallest bf16 result over a dense grid."""
    from scipy.special import lambertw
    ln3 = math.log(3.0)
    zb = _bits(ora, [ln3])
    zv = float(ora.bf16_value(zb)[0])
    got = float(ora.bf16_value(_silu_bf16(ora, zb))[0])
    assert abs(got - 0.75 * ln3) <= 1.1 * abs(zv - ln3) + float(ora.bf16_ulp(np.array([0.75 * ln3]))[0])
    w = float(lambertw(1.0 / math.e).real)
    grid = np.arange(0xBF80, 0xC000, dtype=np.uint16)           # every bf16 in [-2, -1)
    h = ora.bf16_value(_silu_bf16(ora, grid)).astype(np.float64)
    assert abs(h.min() + w) <= float(ora.bf16_ulp(np.array([w]))[0])
    zmin = ora.bf16_value(grid[[np.argmin(h)]])[0]
    assert abs(float(zmin) - (-1.0 - w)) <= 0.05


def test_silu_mul_scaling(ora):
    """h = bf16(silu(g) * u) rounds once: u = 2^j scales h by exactly 2^j (no intermediate rounding of
    silu(g) that the scaling could expose), and u = -1 flips its sign."""
    zb = inputs.activations(86, 1, 128 * 4, outliers=False).ravel()
    base = ora.bf16_value(_silu_bf16(ora, zb)).astype(np.float64)
    for j in (-5, -1, 1, 3, 7):
        h = ora.bf16_value(_silu_bf16(ora, zb, _bits(ora, np.full(zb.size, 2.0 ** j)))).astype(np.float64)
        assert np.array_equal(h, base * 2.0 ** j)
    h = ora.bf16_value(_silu_bf16(ora, zb, _bits(ora, np.full(zb.size, -1.0)))).astype(np.float64)
    assert np.array_equal(h, -base)
