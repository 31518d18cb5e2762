"""A seeded sweep of GEMM shapes across the dispatcher's routes, against the oracle.

The hand-picked parity shapes cover each kernel where it was built to run.  These shapes are drawn
instead: M in four bands (decode widths, 17-64, 65-255, above 255 rows), K/128 small, medium or long,
N/128 small, medium or wide, so that ragged row and column tiles meet K-group counts with and
without the factors the planners divide by.  Each shape runs

  - as the dispatcher routes it, fused (bf16 activations) and on codes, on fragment-order and on
    row-major weights;
  - with the tiled engine forced (up to 255 rows) and with the split-K skinny kernel forced (up to 64
    rows), the two kernels the dispatcher sends only the largest of these shapes to;
  - through the bf16-activation variant where its shape rule admits it (up to 16 rows).

Every result is held to the dense bar against the oracle (|gpu - oracle| <= 1e-2 RMS + 1 bf16 ulp),
on the whole output where the oracle finishes quickly, else on two whole rows and random positions;
the fused call equals the call on codes bit for bit, and the two layouts agree as
`assert_layouts_agree` states.  The host-only test below checks that the draw still reaches every
route the plan query reports, so the sweep keeps its reach when the planners change.
"""
import collections

import numpy as np
import pytest

import inputs
from tests.gpu_util import assert_bits_equal, assert_close, assert_layouts_agree, dev, host, say

SEED = 2026


def draw_shapes(seed=SEED, n=96):
    """(M, K, N) triples, n of them, cycling through the four row bands; N * K is kept at or under
    2^26 so that the oracle's weight quant stays quick."""
    g = np.random.default_rng(seed)
    bands = [(1, 17), (17, 65), (65, 256), (256, 1100)]
    out = []
    for i in range(n):
        lo, hi = bands[i % 4]
        M = int(g.integers(lo, hi))
        kb = g.integers(0, 3)
        G = int(g.integers(1, 9) if kb == 0 else g.integers(9, 48) if kb == 1 else g.choice([56, 64, 96, 112, 128]))
        nb = g.integers(0, 3)
        NT = int(g.integers(1, 9) if nb == 0 else g.integers(9, 64) if nb == 1 else g.choice([96, 112, 128, 256]))
        while NT * G > (1 << 26) // (128 * 128):
            NT = max(1, NT // 2)
        out.append((M, 128 * G, 128 * NT))
    return out


SHAPES = draw_shapes()


def _bf16a_admits(M, K):
    """The bf16-activation entry's shape rule: at most 16 rows, and K/128 = wk * gs with wk <= 8 and
    gs one of 1, 2, 4, 8, 16."""
    G = K // 128
    return M <= 16 and any(G % gs == 0 and G // gs <= 8 for gs in (1, 2, 4, 8, 16))


def test_sweep_reaches_every_route():
    """Host only: the drawn shapes route to the decode kernel with and without a K split, to the
    mid-width kernel with and without one, and to the tiled engine with and without one, on both
    layouts; and some admit the bf16-activation variant."""
    import block_scaled_fp8_r9k_amd as r9k
    r9k.set_dispatch(255, r9k.ENGINE_AUTO)
    for packed in (False, True):
        seen = collections.Counter()
        for M, K, N in SHAPES:
            kern, ks = r9k.gemm_fp8_block_plan(M, K, N, packed)
            seen[(kern, ks > 1)] += 1
        for route in [(r9k.KERNEL_DECODE, False), (r9k.KERNEL_DECODE, True), (r9k.KERNEL_MID, False),
                      (r9k.KERNEL_MID, True), (r9k.KERNEL_TILED, False), (r9k.KERNEL_TILED, True)]:
            assert seen[route] >= 2, (packed, route, dict(seen))
    assert sum(_bf16a_admits(M, K) for M, K, _ in SHAPES) >= 6


@pytest.fixture(scope="module")
def r9k():
    import torch
    import block_scaled_fp8_r9k_amd as m
    assert torch.cuda.is_available()
    m.lib()
    m.set_dispatch(255, m.ENGINE_AUTO)
    yield m
    m.set_dispatch(255, m.ENGINE_AUTO)


def _positions(M, K, N, seed):
    """Every output where the oracle's sum count M*N*K is at most 2^28; else rows 0 and M - 1 whole
    (where N*K is at most 2^25) and 4000 random positions."""
    if M * N * K <= 1 << 28:
        return None
    r = np.random.default_rng(seed)
    rows = np.unique([0, M - 1]) if N * K <= 1 << 25 else np.array([], np.int64)
    ms = np.concatenate([np.repeat(rows, N), r.integers(0, M, 4000)])
    ns = np.concatenate([np.tile(np.arange(N), len(rows)), r.integers(0, N, 4000)])
    return ms, ns


@pytest.mark.gpu
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_sweep_shape(r9k, ora, M, K, N):
    seed = M * 131 + K // 128 * 7 + N // 128
    a = inputs.activations(seed, M, K, outliers=True)
    w = inputs.weights(seed, N, K)
    aq_o, as_o = ora.quant_act(a)
    wq_o, ws_o = ora.quant_weight(w)
    pos = _positions(M, K, N, seed)
    if pos is None:
        _, want = ora.gemm_block(aq_o, as_o, wq_o, ws_o, want_f64=True)
        pick = lambda c: c
    else:
        ms, ns = pos
        _, want = ora.gemm_block_at(aq_o, as_o, wq_o, ws_o, ms, ns, want_f64=True)
        pick = lambda c: c[ms, ns]

    a_d = dev(a)
    wq, ws = r9k.quant_weight(dev(w))
    wp = r9k.pack_weight(wq)
    aq, as_ = r9k.quant_act(a_d)
    results = {}
    for packed in (True, False):
        lay = "packed" if packed else "row-major"
        plan = r9k.gemm_fp8_block_plan(M, K, N, packed)
        say("sweep", M, K, N, lay, "plan", plan)
        if packed:
            fused = host(r9k.gemm_fp8_block_qa_packed(a_d, wp, ws))
            codes = host(r9k.gemm_fp8_block_packed(aq, as_, wp, ws))
        else:
            fused = host(r9k.gemm_fp8_block_qa(a_d, wq, ws))
            codes = host(r9k.gemm_fp8_block(aq, as_, wq, ws))
        assert_close(ora, pick(fused), want, f"{M}x{K}x{N} {lay} plan {plan}")
        assert_bits_equal(fused, codes, f"{M}x{K}x{N} {lay} fused == on codes")
        results[packed] = fused
    assert_layouts_agree(ora, results[True], results[False], f"{M}x{K}x{N} packed vs row-major")

    forced = []
    if M <= 255:
        forced.append(("tiled", r9k.ENGINE_TILED))
    if M <= 64:
        forced.append(("split-K skinny", r9k.ENGINE_SPLITK))
    try:
        for name, engine in forced:
            r9k.set_dispatch(255, engine)
            say("sweep", M, K, N, name, "forced")
            fused = host(r9k.gemm_fp8_block_qa_packed(a_d, wp, ws))
            assert_close(ora, pick(fused), want, f"{M}x{K}x{N} {name} forced")
            assert_bits_equal(fused, host(r9k.gemm_fp8_block_packed(aq, as_, wp, ws)),
                              f"{M}x{K}x{N} {name} forced, fused == on codes")
            assert_bits_equal(fused, host(r9k.gemm_fp8_block_qa(a_d, wq, ws)),
                              f"{M}x{K}x{N} {name} forced, packed == row-major")
    finally:
        r9k.set_dispatch(255, r9k.ENGINE_AUTO)

    if _bf16a_admits(M, K):
        say("sweep", M, K, N, "bf16a")
        got = host(r9k.gemm_fp8_block_bf16a(a_d, wq, ws))
        _, want16 = ora.gemm_block_bf16a(a, host(wq), host(ws), want_f64=True)
        o = np.asarray(want16, np.float64)
        g = ora.bf16_value(got).astype(np.float64)
        bound = ora.bf16_ulp(o) + 1e-5 * float(np.sqrt(np.mean(o * o)))
        err = np.abs(g - o)
        assert np.all(err <= bound), f"bf16a {M}x{K}x{N}: worst {float(np.max(err / bound)):.3f} of the bound"
        assert_bits_equal(host(r9k.gemm_fp8_block_bf16a(a_d, wp, ws, packed=True)), got,
                          f"bf16a {M}x{K}x{N} packed == row-major")
