"""GPU results that must equal the oracle bit for bit, through every engine.

1. Exact sums.  Activations and weights are small integers on the e4m3 grid,
   with one +-448 in every activation group and every 128x128 weight block, so
   that every group and block scale is exactly 1 and quantisation is the
   identity.  Each +-448 meets a zero on the other side (position 0 of every
   group: the activation's +-448 against zero weights; position 1: the
   weight's 448 against zero activations), so every nonzero product is an
   integer of magnitude at most 256 and every partial sum stays below 2^20: the
   GPU's accumulation (MFMA sums, promotion, K-split partials) is then exact.
   (With 448 x 448 products beside small ones it is not: the fp8 MFMA's
   internal 128-term sum is not an IEEE fp32 sum, and a few outputs in 10^5
   then land one bf16 ulp off.)  What remains is the one rounding of the exact
   integer to bf16, which must be round-to-nearest-even: truncation (or any
   other rounding) would change about half of the outputs, which the test
   also checks.
2. Adversarial activation groups (all +0, all -0, subnormal-only, a single
   value, powers of two, e4m3 midpoints, a maximum at either end, ...) through
   every in-load quant: the fused call must equal the split call (r9k_quant_act,
   pinned bit-exact against the oracle, then the GEMM on codes) bit for bit,
   and each row must meet the oracle to the tolerance.
"""
import numpy as np
import pytest

import inputs
from tests.gpu_util import assert_bits_equal, assert_close, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def r9k():
    import torch
    import block_scaled_fp8_r9k_amd as m
    assert torch.cuda.is_available()
    m.lib()
    m.set_dispatch(255, m.ENGINE_AUTO)
    yield m
    m.set_dispatch(255, m.ENGINE_AUTO)


def _int_grid(rng, shape):
    """Integers in [-16, 16]: all exactly representable in e4m3 (and bf16)."""
    return rng.integers(-16, 17, size=shape).astype(np.float32)


def exact_operands(seed, M, K, N):
    rng = np.random.default_rng(seed)
    a = _int_grid(rng, (M, K))
    w = _int_grid(rng, (N, K))
    for g in range(K // 128):
        # position 0: every activation group's +-448, against zero weights
        a[:, g * 128] = np.where(rng.integers(0, 2, M) == 1, 448.0, -448.0)
        w[:, g * 128] = 0.0
        # position 1: every weight block's 448 (one row of the block), against zero activations
        a[:, g * 128 + 1] = 0.0
        w[:, g * 128 + 1] = _int_grid(rng, N)
        for bn in range(N // 128):
            w[bn * 128 + rng.integers(0, 128), g * 128 + 1] = 448.0
    return inputs.to_bf16_bits(a), inputs.to_bf16_bits(w)


def _truncated(c64):
    """bf16 bits of the exact (integer, < 2^24, so exact in fp32) values truncated toward zero."""
    return (np.asarray(c64, np.float32).view(np.uint32) >> 16).astype(np.uint16)


# (M, K, N, the kernel the plan must name, whether it splits K)
ROUTES = [
    (4, 4096, 2048, "decode", False),
    (16, 14336, 2048, "decode", True),
    (32, 4096, 4096, "mid", False),
    (128, 4096, 4096, "mid", False),
    (255, 4096, 4096, "mid", False),
    (32, 14336, 4096, "mid", True),
    (16, 8192, 32768, "mid", True),
    (256, 4096, 4096, "tiled", True),
    (512, 256, 2048, "tiled", False),
]
KERNELS = {"decode": 1, "skinny": 2, "tiled": 3, "mid": 4}


@pytest.mark.parametrize("M,K,N,kern,split", ROUTES + [(16, 2048, 4096, "skinny", True), (4, 4096, 2048, "skinny", True)])
def test_exact_sums_round_to_nearest_even(r9k, ora, M, K, N, kern, split):
    # the split-K skinny kernel is taken by the dispatcher only for large K and N below 8 rows; here it
    # is forced (R9K_ENGINE_SPLITK) at shapes the oracle handles quickly
    r9k.set_dispatch(255, r9k.ENGINE_SPLITK if kern == "skinny" else r9k.ENGINE_AUTO)
    try:
        _exact_sums(r9k, ora, M, K, N, kern, split)
    finally:
        r9k.set_dispatch(255, r9k.ENGINE_AUTO)


def _exact_sums(r9k, ora, M, K, N, kern, split):
    for packed in (False, True):
        k, ks = r9k.gemm_fp8_block_plan(M, K, N, packed)
        assert k == KERNELS[kern] and (ks > 1) == split, (packed, k, ks)
    say("exact sums", M, K, N, kern)
    a, w = exact_operands(M + N, M, K, N)
    wq_o, ws_o = ora.quant_weight(w)
    aq_o, as_o = ora.quant_act(a)
    assert np.all(ws_o == 1.0) and np.all(as_o == 1.0), "the construction gives unit scales"
    c_o, c64 = ora.gemm_block(aq_o, as_o, wq_o, ws_o, want_f64=True)
    assert np.all(np.abs(c64) < 2.0 ** 20) and np.array_equal(c64, np.round(c64))
    differs = np.count_nonzero(_truncated(c64) != c_o)
    assert differs > c_o.size // 4, f"only {differs} of {c_o.size} outputs tell RNE from truncation"
    a_d = dev(a)
    wq, ws = r9k.quant_weight(dev(w))
    wp = r9k.pack_weight(wq)
    aq, as_ = r9k.quant_act(a_d)
    for name, got in (("fused", r9k.gemm_fp8_block_qa(a_d, wq, ws)),
                      ("split", r9k.gemm_fp8_block(aq, as_, wq, ws)),
                      ("fused packed", r9k.gemm_fp8_block_qa_packed(a_d, wp, ws)),
                      ("split packed", r9k.gemm_fp8_block_packed(aq, as_, wp, ws))):
        assert_bits_equal(host(got), c_o, f"{kern} {name} {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N", [(1, 4096, 2048), (8, 4096, 2048), (16, 2048, 1024)])
def test_exact_sums_bf16a(r9k, ora, M, K, N):
    """The bf16-activation variant on integer activations: the same exact-sum argument without any
    activation quant."""
    say("exact sums bf16a", M, K, N)
    a, w = exact_operands(M * 3 + N, M, K, N)
    wq_o, ws_o = ora.quant_weight(w)
    c_o, c64 = ora.gemm_block_bf16a(a, wq_o, ws_o, want_f64=True)
    assert np.array_equal(c64, np.round(c64)) and np.all(np.abs(c64) < 2.0 ** 20)
    assert np.count_nonzero(_truncated(c64) != c_o) > c_o.size // 4
    wq, ws = r9k.quant_weight(dev(w))
    assert_bits_equal(host(r9k.gemm_fp8_block_bf16a(dev(a), wq, ws)), c_o, "bf16a")
    assert_bits_equal(host(r9k.gemm_fp8_block_bf16a(dev(a), r9k.pack_weight(wq), ws, packed=True)), c_o,
                      "bf16a packed")


def edge_rows(M, K):
    """M rows of K bf16 values built from the adversarial groups: rows 0-11 repeat one kind of group along
    K, the others cycle through all kinds with a row-dependent rotation."""
    edge = inputs.quant_edge_groups().reshape(-1, 128)
    kinds = edge.shape[0]
    G = K // 128
    rows = np.empty((M, K), np.uint16)
    for r in range(M):
        for g in range(G):
            kind = r % kinds if r < kinds else (r + g) % kinds
            rows[r, g * 128:(g + 1) * 128] = edge[kind]
    return rows


@pytest.mark.parametrize("M,K,N,kern", [(12, 1536, 2048, "decode"), (40, 1536, 6144, "decode"),
                                        (16, 15360, 2048, "decode"), (16, 2048, 4096, "skinny")])
def test_inload_quant_edge_groups(r9k, ora, M, K, N, kern):
    """Every in-load quant (the decode kernel's four lanes a group, with and without a K split, and the
    skinny kernel's sixteen, forced) on the adversarial groups: fused == split bit for bit on both weight
    layouts, each row to the tolerance."""
    r9k.set_dispatch(255, r9k.ENGINE_SPLITK if kern == "skinny" else r9k.ENGINE_AUTO)
    try:
        _edge_groups(r9k, ora, M, K, N, kern)
    finally:
        r9k.set_dispatch(255, r9k.ENGINE_AUTO)


def _edge_groups(r9k, ora, M, K, N, kern):
    for packed in (False, True):
        assert r9k.gemm_fp8_block_plan(M, K, N, packed)[0] == KERNELS[kern]
    say("edge groups", M, K, N, kern)
    a = edge_rows(M, K)
    w = inputs.weights(M + 5, N, K)
    wq_o, ws_o = ora.quant_weight(w)
    aq_o, as_o = ora.quant_act(a)
    a_d = dev(a)
    wq, ws = r9k.quant_weight(dev(w))
    wp = r9k.pack_weight(wq)
    aq, as_ = r9k.quant_act(a_d)
    assert_bits_equal(host(aq), aq_o, "edge codes")
    assert_bits_equal(host(as_), as_o, "edge scales")
    fused = host(r9k.gemm_fp8_block_qa(a_d, wq, ws))
    assert_bits_equal(fused, host(r9k.gemm_fp8_block(aq, as_, wq, ws)), f"{kern} fused == split")
    fused_p = host(r9k.gemm_fp8_block_qa_packed(a_d, wp, ws))
    assert_bits_equal(fused_p, host(r9k.gemm_fp8_block_packed(aq, as_, wp, ws)), f"{kern} packed fused == split")
    rows = np.unique(np.concatenate([np.arange(min(M, 12)), [M - 1]]))
    ns = np.arange(N)
    for r in rows:
        _, c64 = ora.gemm_block_at(aq_o, as_o, wq_o, ws_o, np.full(N, r), ns, want_f64=True)
        assert_close(ora, fused[r], c64, f"{kern} edge row {r}")
        assert_close(ora, fused_p[r], c64, f"{kern} packed edge row {r}")


def test_moe_gateup_inload_quant_edge_groups(r9k, ora):
    """The MoE gate_up kernel quantises x in its A-load: edge-group tokens against the oracle's gu
    (three-launch path, which stores gu), token by token, and the fused path against the three-launch
    path bit for bit.  The huge group (1e30) is left out of x here: silu(gate) * up of such a token
    overflows fp32 before h is re-quantised, which no decode input reaches."""
    import torch
    T, H, E, I, k = 11, 1536, 3, 256, 2
    edge = inputs.quant_edge_groups().reshape(-1, 128)
    edge = np.delete(edge, 10, axis=0)           # the group holding 1e30
    x = np.empty((T, H), np.uint16)
    for t in range(T):
        for g in range(H // 128):
            x[t, g * 128:(g + 1) * 128] = edge[(t + g) % edge.shape[0]] if t else edge[g % edge.shape[0]]
    _, logits, w13, w2 = inputs.moe_inputs(7, T, H, E, I)
    ids, tw = ora.moe_route(logits, k)
    q13 = [ora.quant_weight(w13[e]) for e in range(E)]
    q2 = [ora.quant_weight(w2[e]) for e in range(E)]
    o13 = (np.stack([a for a, _ in q13]), np.stack([b for _, b in q13]))
    o2 = (np.stack([a for a, _ in q2]), np.stack([b for _, b in q2]))
    _, inter = ora.moe_decode(x, ids, tw, o13[0], o13[1], o2[0], o2[1], intermediates=True)
    g13, s13 = r9k.quant_weight(dev(w13.reshape(E * 2 * I, H)))
    g2, s2 = r9k.quant_weight(dev(w2.reshape(E * H, I)))
    args = (dev(x), dev(ids), dev(tw), g13.view(E, 2 * I, H), s13.view(E, 2 * I // 128, H // 128),
            g2.view(E, H, I), s2.view(E, H // 128, I // 128))
    ws = torch.zeros(r9k.moe_fp8_decode_workspace(T, H, E, I, k), dtype=torch.uint8, device="cuda")
    say("moe edge groups")
    unfused = host(r9k.moe_fp8_decode(*args, workspace=ws, fused=False))
    off = r9k.moe_ws_offset(T, H, E, I, k, "gu")
    gu = host(ws[off:off + T * k * 2 * I * 2].view(torch.bfloat16).view(T * k, 2 * I))
    gu_o = ora.bf16_value(inter["gu"]).astype(np.float64)
    for p in range(T * k):
        assert_close(ora, gu[p], gu_o[p], f"moe gu, pair {p}")
    fused = host(r9k.moe_fp8_decode(*args, workspace=ws, fused=True))
    assert_bits_equal(fused, unfused, "moe fused == three-launch on edge tokens")
