"""Fragment-order weights (r9k_pack_weight and the _packed GEMMs).

The packed layout is checked byte for byte against its definition, restated
here with numpy.  The GEMMs on packed weights must equal the row-major GEMMs
on the same codes bit for bit whenever the two run the same launch (the kernels
receive the same register contents), in both the fused and the split form; the
decode kernel's planner may slice K differently for the two layouts (each
layout's fastest launch), and then they agree up to the fp32 summation order
(within one bf16 ulp, on a small share of the outputs).  The row-major GEMMs
are the ones pinned to the oracle (test_gpu_gemm.py).
"""
import numpy as np
import pytest

import inputs
from tests.gpu_util import assert_bits_equal, assert_close, assert_layouts_agree, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def r9k():
    import torch
    import block_scaled_fp8_r9k_amd as r9k
    assert torch.cuda.is_available()
    r9k.lib()
    yield r9k
    r9k.set_dispatch(255, r9k.ENGINE_AUTO)


def pack_reference(wq: np.ndarray) -> np.ndarray:
    """The layout's definition: block (t, g) at (t * G + g) * 2048 holds, at
    h * 1024 + 16 l, row 16 t + l % 16, bytes 128 g + 64 h + 16 (l // 16) .. +15."""
    N, K = wq.shape
    G = K // 128
    x = wq.reshape(N // 16, 16, G, 2, 4, 16)      # t, r, g, h, q, byte
    x = x.transpose(0, 2, 3, 4, 1, 5)             # t, g, h, q, r, byte  (lane = 16 q + r)
    return np.ascontiguousarray(x).reshape(N, K)


def test_pack_layout(r9k):
    rng = np.random.default_rng(7)
    for N, K in ((128, 128), (256, 384), (1024, 512)):
        wq = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
        got = host(r9k.pack_weight(dev(wq)))
        assert_bits_equal(got, pack_reference(wq), f"pack {N}x{K}")


def test_pack_rejects_overlap(r9k):
    import torch
    w = torch.zeros((256, 256), dtype=torch.uint8, device="cuda")
    with pytest.raises(r9k.R9kError):
        r9k.pack_weight(w, wp=w)


@pytest.mark.parametrize("M,K,N", [(1, 512, 1024), (4, 4096, 1024), (16, 1024, 384), (17, 256, 640),
                                   (100, 384, 384), (255, 512, 256), (256, 512, 256), (300, 256, 384),
                                   (600, 1024, 1152)])
@pytest.mark.parametrize("engine", [0, 1, 2])
def test_packed_equals_row_major(r9k, ora, M, K, N, engine):
    say("packed", M, K, N, engine)
    a = dev(inputs.activations(M, M, K))
    wq, ws = r9k.quant_weight(dev(inputs.weights(M, N, K)))
    wp = r9k.pack_weight(wq)
    r9k.set_dispatch(255, engine)
    # the decode kernel may take another K slicing on each layout; every other launch is the same
    decode = r9k.gemm_fp8_block_plan(M, K, N, False)[0] == r9k.KERNEL_DECODE
    same = assert_layouts_agree if decode else (lambda ora_, x, y, what: assert_bits_equal(x, y, what))
    ref = host(r9k.gemm_fp8_block_qa(a, wq, ws))
    same(ora, host(r9k.gemm_fp8_block_qa_packed(a, wp, ws)), ref, f"fused {M}x{K}x{N} e{engine}")
    aq, as_ = r9k.quant_act(a)
    ref_s = host(r9k.gemm_fp8_block(aq, as_, wq, ws))
    same(ora, host(r9k.gemm_fp8_block_packed(aq, as_, wp, ws)), ref_s, f"split {M}x{K}x{N} e{engine}")


def test_packed_decode_sweep_against_oracle(r9k, ora):
    """The benchmark's decode shapes on packed weights, every output against the oracle."""
    K, N = 4096, 14336
    a_bits = inputs.activations(0, 16, K, outliers=True)
    w_bits = inputs.weights(0, N, K)
    wq_o, ws_o = ora.quant_weight(w_bits)
    wq, ws = r9k.quant_weight(dev(w_bits))
    wp = r9k.pack_weight(wq)
    r9k.set_dispatch(255, 0)
    for M in (1, 2, 4, 8, 16):
        say("packed decode", M)
        aq_o, as_o = ora.quant_act(a_bits[:M])
        _, c64 = ora.gemm_block(aq_o, as_o, wq_o, ws_o, want_f64=True)
        got = host(r9k.gemm_fp8_block_qa_packed(dev(a_bits[:M]), wp, ws))
        assert_close(ora, got, c64, f"packed decode M={M}")
