"""GPU parity for the mid-width kernel (17 to 256 rows) through the C ABI: all of K per CTA on
activations quantised once per call, or, at long K and up to 64 rows, a K split of 4 or 8 whose fp32
partials a second launch sums in ascending split order (20 x 14336, 48 x 8192, 40 x 14336 at N = 2048,
64 x 12288).  The shapes cover every planned configuration kind: one to four row tiles (a last row block
holding fewer rows than its tile), one column tile per CTA with K split over eight, four or one waves,
two and four column tiles per CTA sharing staged activations, and load rings of one, two and four steps.
Every output is checked against the oracle; the fused call equals the split call, and the two weight
layouts give the same bits (the same launch)."""
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


@pytest.mark.parametrize("M,K,N", [(17, 4096, 4096), (20, 14336, 4096), (17, 1152, 4096), (33, 3072, 4096),
                                   (40, 2048, 4096), (48, 2048, 16384), (60, 4096, 4096), (64, 2048, 8192),
                                   (130, 1024, 4096), (128, 2048, 4096), (200, 1536, 4096), (255, 512, 4096),
                                   (100, 384, 4096), (70, 640, 1024), (255, 512, 256), (255, 768, 4096),
                                   (48, 8192, 4096), (40, 14336, 2048), (64, 12288, 4096), (130, 8192, 1024)])
def test_mid_against_oracle(r9k, ora, M, K, N):
    plans = {r9k.gemm_fp8_block_plan(M, K, N, packed) for packed in (False, True)}
    assert len(plans) == 1
    kernel, ksplit = plans.pop()
    assert kernel == r9k.KERNEL_MID and (K // 128) % ksplit == 0
    say("mid", M, K, N, "ksplit", ksplit)
    a = inputs.activations(M + 1, M, K, outliers=True)
    w = inputs.weights(K // 128, N, K)
    wq_o, ws_o = ora.quant_weight(w)
    aq_o, as_o = ora.quant_act(a)
    _, c64 = ora.gemm_block(aq_o, as_o, wq_o, ws_o, want_f64=True)
    a_d = dev(a)
    wq, ws = r9k.quant_weight(dev(w))
    wp = r9k.pack_weight(wq)
    fused = host(r9k.gemm_fp8_block_qa(a_d, wq, ws))
    assert_close(ora, fused, c64, f"mid {M}x{K}x{N}")
    aq, as_ = r9k.quant_act(a_d)
    assert_bits_equal(host(r9k.gemm_fp8_block(aq, as_, wq, ws)), fused, "mid split == fused")
    assert_bits_equal(host(r9k.gemm_fp8_block_qa_packed(a_d, wp, ws)), fused, "mid packed == row-major")
    assert_bits_equal(host(r9k.gemm_fp8_block_packed(aq, as_, wp, ws)), fused, "mid split packed")
    assert_bits_equal(host(r9k.gemm_fp8_block_qa(a_d, wq, ws)), fused, "mid repeat")
