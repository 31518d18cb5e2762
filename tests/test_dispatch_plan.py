"""The dispatcher's decision on the host: which kernel a GEMM call of a given
shape runs, with its K split, through r9k_gemm_fp8_block_plan (launches
nothing, needs no device).  The workspace the library asks for must cover the
fp32 partials of every K split it plans.
"""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def r9k():
    import block_scaled_fp8_r9k_amd as m
    m.set_dispatch(255, m.ENGINE_AUTO)
    yield m
    m.set_dispatch(255, m.ENGINE_AUTO)


def test_kernel_codes_match_header(r9k):
    text = open(os.path.join(ROOT, "include", "r9k.h")).read()
    d = {k: int(v) for k, v in re.findall(r"#define\s+(R9K_KERNEL_\w+)\s+(\d+)", text)}
    assert d == {"R9K_KERNEL_NONE": r9k.KERNEL_NONE, "R9K_KERNEL_DECODE": r9k.KERNEL_DECODE,
                 "R9K_KERNEL_SKINNY": r9k.KERNEL_SKINNY, "R9K_KERNEL_TILED": r9k.KERNEL_TILED,
                 "R9K_KERNEL_MID": r9k.KERNEL_MID}


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("M", list(range(1, 17)))
def test_decode_sweep_streams_whole_rows(r9k, M, packed):
    # single-token to 16-row decode on the 4096 -> 14336 projection: one pass
    # over the weight, no K split (at 10 and 11 rows half-width CTAs would pass
    # the repeated-quant budget and split K; the wide CTAs from 9 rows on do not)
    assert r9k.gemm_fp8_block_plan(M, 4096, 14336, packed) == (r9k.KERNEL_DECODE, 1)
    assert r9k.gemm_fp8_block_plan(M, 4096, 12288, packed) == (r9k.KERNEL_DECODE, 1)


@pytest.mark.parametrize("M,K,N", [(16, 14336, 4096), (8, 14336, 4096), (16, 14336, 2048), (1, 28672, 1024)])
def test_decode_k_split(r9k, M, K, N):
    for packed in (False, True):
        kern, ks = r9k.gemm_fp8_block_plan(M, K, N, packed)
        assert kern == r9k.KERNEL_DECODE and ks >= 2, (M, K, N, packed, kern, ks)
        assert (K // 128) % ks == 0


@pytest.mark.parametrize("M,K,N", [(256, 4096, 4096), (300, 4096, 4096), (4096, 4096, 12288), (255, 14336, 4096),
                                   (129, 8192, 4096), (65, 14336, 4096), (128, 14336, 4096), (65, 8192, 4096),
                                   (65, 4096, 14336), (255, 4096, 14336), (129, 4096, 8192), (129, 4096, 6144),
                                   (255, 512, 8192)])
def test_wide_shapes_go_tiled(r9k, M, K, N):
    # above 255 rows; and above 64 rows at long K or where the mid-width kernel's 64 x 64 blocks would
    # need more than one CTA per compute unit (ceil(M / 64) * N / 64 > 256)
    kern, ks = r9k.gemm_fp8_block_plan(M, K, N)
    assert kern == r9k.KERNEL_TILED and ks >= 1


@pytest.mark.parametrize("M,K,N", [(17, 4096, 4096), (32, 4096, 4096), (64, 4096, 4096), (128, 4096, 4096),
                                   (255, 4096, 4096), (32, 14336, 4096), (64, 14336, 4096), (48, 4096, 16384),
                                   (32, 4096, 65536), (64, 4096, 14336), (33, 4096, 14336), (128, 4096, 8192),
                                   (128, 4096, 6144), (200, 4096, 4096), (255, 512, 4096)])
def test_mid_widths_run_in_one_launch(r9k, M, K, N):
    # 17 to 255 rows where the decode kernel would need a K split: the mid-width kernel, all of K per
    # CTA (one launch after the activation quant), except up to 64 rows at long K, where its K split of
    # 64-column blocks and the ordered reduce launch move fewer bytes per compute unit; above 64 rows
    # only at K < 8192 and where its 64 x 64 blocks fit one CTA per compute unit
    split = M <= 64 and K >= 8192
    for packed in (False, True):
        kern, ks = r9k.gemm_fp8_block_plan(M, K, N, packed)
        assert kern == r9k.KERNEL_MID, (M, K, N, kern)
        assert (ks > 1) == split and (K // 128) % ks == 0 and (N // 64) * ks >= 256 if split else ks == 1, ks


def test_prefill_has_no_k_split(r9k):
    # 16 x 48 tiles of 256 x 256 already fill the chip
    assert r9k.gemm_fp8_block_plan(4096, 4096, 12288) == (r9k.KERNEL_TILED, 1)


def test_empty_call_plans_nothing(r9k):
    assert r9k.gemm_fp8_block_plan(0, 4096, 4096) == (r9k.KERNEL_NONE, 0)


def test_forced_engines(r9k):
    try:
        r9k.set_dispatch(255, r9k.ENGINE_TILED)
        assert r9k.gemm_fp8_block_plan(1, 4096, 14336)[0] == r9k.KERNEL_TILED
        r9k.set_dispatch(0, r9k.ENGINE_AUTO)           # the skinny engine takes no width
        assert r9k.gemm_fp8_block_plan(1, 4096, 14336)[0] == r9k.KERNEL_TILED
        r9k.set_dispatch(255, r9k.ENGINE_SKINNY)
        # shapes the decode kernel does not take without a K split: the mid-width kernel up to 256 rows,
        # the split-K skinny kernel above
        assert r9k.gemm_fp8_block_plan(200, 4096, 4096)[0] == r9k.KERNEL_MID
        assert r9k.gemm_fp8_block_plan(300, 4096, 4096)[0] == r9k.KERNEL_SKINNY
        assert r9k.gemm_fp8_block_plan(4, 4096, 4096)[0] == r9k.KERNEL_DECODE
    finally:
        r9k.set_dispatch(255, r9k.ENGINE_AUTO)


@pytest.mark.parametrize("M", [1, 5, 16, 17, 32, 48, 64, 65, 100, 128, 200, 255, 256, 300, 1024])
@pytest.mark.parametrize("K,N", [(4096, 4096), (14336, 4096), (4096, 14336), (512, 1024), (1280, 384)])
def test_workspace_covers_partials(r9k, M, K, N):
    ws = r9k.gemm_fp8_block_workspace(M, K, N)
    for packed in (False, True):
        kern, ks = r9k.gemm_fp8_block_plan(M, K, N, packed)
        assert kern in (r9k.KERNEL_DECODE, r9k.KERNEL_SKINNY, r9k.KERNEL_TILED, r9k.KERNEL_MID)
        assert 1 <= ks <= K // 128
        if ks > 1:
            assert ws >= 4 * ks * M * N, (M, K, N, packed, ks, ws)
        if kern in (r9k.KERNEL_MID, r9k.KERNEL_TILED):   # activation codes and scales, quantised once a call
            assert ws >= M * K + 4 * M * (K // 128), (M, K, N, packed, ws)


def test_random_shapes_plan_valid_splits(r9k):
    """Seeded random shapes (1-600 rows, K up to 32768, N up to 65536) through every planner: the plan
    query succeeds on both layouts, a K split fits K/128, and the workspace the library asks for holds
    the split's fp32 partials and, for the kernels that read codes quantised once a call, the codes and
    scales."""
    import numpy as np
    g = np.random.default_rng(11)
    for _ in range(3000):
        M = int(g.integers(1, 601))
        K = 128 * int(g.choice([g.integers(1, 33), g.integers(33, 257)]))
        N = 128 * int(g.choice([g.integers(1, 65), g.integers(65, 513)]))
        ws = r9k.gemm_fp8_block_workspace(M, K, N)
        for packed in (False, True):
            kern, ks = r9k.gemm_fp8_block_plan(M, K, N, packed)
            assert kern in (r9k.KERNEL_DECODE, r9k.KERNEL_SKINNY, r9k.KERNEL_TILED, r9k.KERNEL_MID), (M, K, N)
            # the tiled kernel hands split s the groups [s G / S, (s + 1) G / S), so any S up to G
            # will do; the other kernels' splits take equal K ranges
            assert 1 <= ks <= K // 128, (M, K, N, packed, kern, ks)
            if kern != r9k.KERNEL_TILED:
                assert (K // 128) % ks == 0, (M, K, N, packed, kern, ks)
            if M > 255:
                assert kern == r9k.KERNEL_TILED, (M, K, N, packed, kern)
            if ks > 1:
                assert ws >= 4 * ks * M * N, (M, K, N, packed, kern, ks, ws)
            if kern in (r9k.KERNEL_MID, r9k.KERNEL_TILED):
                assert ws >= M * K + 4 * M * (K // 128), (M, K, N, packed, ws)


def test_plan_argument_checks(r9k):
    L = r9k.lib()
    from ctypes import byref, c_int
    k, s = c_int(), c_int()
    assert L.r9k_gemm_fp8_block_plan(1, 4096, 4096, 0, None, byref(s)) == -1
    assert L.r9k_gemm_fp8_block_plan(1, 4000, 4096, 0, byref(k), byref(s)) == -2
    assert L.r9k_gemm_fp8_block_plan(1, 4096, 4000, 0, byref(k), byref(s)) == -2
    assert L.r9k_gemm_fp8_block_plan(-1, 4096, 4096, 0, byref(k), byref(s)) == -2
    assert L.r9k_gemm_fp8_block_plan(1, 4096, 4096, 2, byref(k), byref(s)) == -7


@pytest.mark.parametrize("M,K,N", [(1, 4096, 128256), (4, 4096, 128256), (8, 4096, 151936), (16, 4096, 151936),
                                   (8, 4096, 32768), (16, 4096, 28672)])
def test_wide_n_decode_streams_whole_rows(r9k, M, K, N):
    # very wide outputs (an LM head over a large vocabulary) at decode widths: every CTA repeats the
    # activation quant, but at most a quarter as many values as the weight bytes it streams, so the decode
    # kernel covers all of K in one launch
    for packed in (False, True):
        assert r9k.gemm_fp8_block_plan(M, K, N, packed) == (r9k.KERNEL_DECODE, 1), (M, K, N, packed)


@pytest.mark.parametrize("M,K,N,kern", [(128, 8192, 2048, 4), (255, 8192, 1024, 4), (192, 14336, 1024, 4),
                                        (128, 14336, 2048, 3), (128, 8192, 3072, 3), (255, 8192, 4096, 3)])
def test_long_k_above_64_rows(r9k, M, K, N, kern):
    # above 64 rows at K >= 8192 the tiled engine only for weights past 2^24 bytes; narrower weights would
    # need its K split 8 to 32 ways, and the mid-width kernel streams them faster
    for packed in (False, True):
        assert r9k.gemm_fp8_block_plan(M, K, N, packed)[0] == kern, (M, K, N, packed)


@pytest.mark.parametrize("M,K,N,split", [(8, 14336, 2048, True), (12, 8192, 1024, True), (6, 16384, 2048, True),
                                         (4, 14336, 2048, False), (8, 8192, 2048, False), (16, 4096, 2048, False)])
def test_decode_few_ctas_split_at_long_k(r9k, M, K, N, split):
    # a whole-K grid of fewer than 192 CTAs at K >= 8192 takes the K split once each CTA would
    # re-quantise 12 x 8192 activation values or more
    for packed in (False, True):
        kern, ks = r9k.gemm_fp8_block_plan(M, K, N, packed)
        assert kern == r9k.KERNEL_DECODE and (ks > 1) == split, (M, K, N, packed, kern, ks)


@pytest.mark.parametrize("M,K,N", [(12, 4096, 6144), (16, 4096, 6144), (12, 4096, 11008), (16, 4096, 11008),
                                   (16, 2048, 6144)])
def test_decode_wide_ctas_keep_whole_rows(r9k, M, K, N):
    # from 5 rows two or four column tiles a CTA down to 168 CTAs: the CTAs repeat the activation quant
    # fewer times, which keeps these shapes under the quant budget and off the K split
    for packed in (False, True):
        assert r9k.gemm_fp8_block_plan(M, K, N, packed) == (r9k.KERNEL_DECODE, 1), (M, K, N, packed)


@pytest.mark.parametrize("M,K,N,kern", [(17, 4096, 14336, 1), (24, 2048, 14336, 1), (64, 512, 14336, 1),
                                        (32, 1024, 4096, 1), (17, 512, 1024, 1),
                                        (17, 4096, 2048, 4), (32, 4096, 2048, 4), (64, 2048, 2048, 4),
                                        (48, 1024, 4096, 4), (32, 4096, 28672, 4), (64, 2048, 28672, 4)])
def test_whole_k_decode_against_mid_from_17_rows(r9k, M, K, N, kern):
    # from 17 rows, where the decode kernel covers all of K per CTA, the lower of the two estimated
    # times: the decode kernel keeps shapes whose busiest compute unit streams many weight bytes next to
    # the activations it re-quantises (N = 14336, or short K); with few column tiles a CTA, or two CTAs
    # a compute unit at K >= 2048, the mid-width kernel on activations quantised once is faster
    want = r9k.KERNEL_DECODE if kern == 1 else r9k.KERNEL_MID
    for packed in (False, True):
        assert r9k.gemm_fp8_block_plan(M, K, N, packed) == (want, 1), (M, K, N, packed)


@pytest.mark.parametrize("M,K,N", [(8, 16384, 32768), (12, 8192, 32768), (16, 8192, 32768), (16, 16384, 16384)])
def test_large_k_and_n_from_8_rows_go_mid(r9k, M, K, N):
    # large K and N at 8 to 16 rows, where the decode kernel fits neither way: the mid-width kernel with
    # its K split
    for packed in (False, True):
        kern, ks = r9k.gemm_fp8_block_plan(M, K, N, packed)
        assert kern == r9k.KERNEL_MID and ks > 1, (packed, kern, ks)


def test_forced_split_k_engine(r9k):
    # R9K_ENGINE_SPLITK: the split-K skinny kernel up to the boundary, the tiled engine above it
    r9k.set_dispatch(255, r9k.ENGINE_SPLITK)
    try:
        assert r9k.gemm_fp8_block_plan(16, 2048, 4096)[0] == r9k.KERNEL_SKINNY
        assert r9k.gemm_fp8_block_plan(255, 1024, 1024)[0] == r9k.KERNEL_SKINNY
        assert r9k.gemm_fp8_block_plan(256, 1024, 1024)[0] == r9k.KERNEL_TILED
    finally:
        r9k.set_dispatch(255, r9k.ENGINE_AUTO)


@pytest.mark.parametrize("M,K,N", [(4, 16384, 65536), (2, 16384, 131072)])
def test_wide_n_goes_to_the_skinny_kernel(r9k, M, K, N):
    # large K and N below 8 rows, where the decode kernel does not fit all of K per CTA (its LDS holds
    # M x K codes): the skinny kernel, with its quant in the A-load
    for packed in (False, True):
        kern, ks = r9k.gemm_fp8_block_plan(M, K, N, packed)
        assert kern == r9k.KERNEL_SKINNY and ks >= 1, (packed, kern, ks)
