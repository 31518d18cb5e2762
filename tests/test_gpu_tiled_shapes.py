"""The tiled engine's tile shapes and K splits, each forced, against the oracle.

Shapes cover ragged M, a last column tile half full (N % 256 == 128), K
splits that divide the group count unevenly (K = 896: 7 groups), and both
weight layouts; every output is compared with the oracle to the GEMM bar.
"""
import numpy as np
import pytest

import inputs
from tests.gpu_util import assert_bits_equal, assert_close, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def r9k():
    import torch
    import block_scaled_fp8_r9k_amd as r9k
    assert torch.cuda.is_available()
    r9k.lib()
    yield r9k
    r9k.set_dispatch(255, r9k.ENGINE_AUTO)
    r9k.set_tiled_plan(r9k.TILE_AUTO, 0)


@pytest.fixture(scope="module")
def problems(r9k, ora):
    out = {}
    for M, K, N in ((77, 896, 384), (200, 896, 640), (300, 1024, 384), (513, 640, 896)):
        a = inputs.activations(M + K, M, K)
        w = inputs.weights(M + N, N, K)
        wq_o, ws_o = ora.quant_weight(w)
        aq_o, as_o = ora.quant_act(a)
        _, c64 = ora.gemm_block(aq_o, as_o, wq_o, ws_o, want_f64=True)
        wq, ws = r9k.quant_weight(dev(w))
        out[(M, K, N)] = (dev(a), wq, r9k.pack_weight(wq), ws, c64)
    return out


@pytest.mark.parametrize("shape", ["256x128", "256x256", "128x64", "256x64"])
@pytest.mark.parametrize("ksplit", [1, 3, 7])
def test_tiled_shape_and_split(r9k, ora, problems, shape, ksplit):
    code = {"256x256": r9k.TILE_256X256, "256x128": r9k.TILE_256X128, "128x64": r9k.TILE_128X64,
            "256x64": r9k.TILE_256X64}[shape]
    r9k.set_tiled_plan(code, ksplit)
    r9k.set_dispatch(255, r9k.ENGINE_TILED)
    try:
        for (M, K, N) in problems:
            # the plan the call runs: the forced split (none for the 256 x 256 tile), clamped to K/128
            want = 1 if shape == "256x256" else min(ksplit, K // 128)
            assert r9k.gemm_fp8_block_plan(M, K, N) == (r9k.KERNEL_TILED, want), (shape, ksplit, M, K, N)
        for (M, K, N), (a, wq, wp, ws, c64) in problems.items():
            say("tiled", shape, ksplit, M, K, N)
            got = host(r9k.gemm_fp8_block_qa(a, wq, ws))
            assert_close(ora, got, c64, f"tiled {shape} ksplit={ksplit} {M}x{K}x{N}")
            assert_bits_equal(host(r9k.gemm_fp8_block_qa_packed(a, wp, ws)), got, "packed == row-major")
            aq, as_ = r9k.quant_act(a)
            assert_bits_equal(host(r9k.gemm_fp8_block(aq, as_, wq, ws)), got, "split == fused")
    finally:
        r9k.set_tiled_plan(r9k.TILE_AUTO, 0)
        r9k.set_dispatch(255, r9k.ENGINE_AUTO)
