"""The allocation-free entry point r9k_gemm_fp8_block_qa_noalloc, through the C ABI, against the existing
r9k_gemm_fp8_block_qa (same kernels, caller's workspace): bit for bit, on two calls in a row, the second with
a smaller input, for both weight layouts; and its scratch limit is enforced."""
import ctypes
from ctypes import c_void_p

import numpy as np
import pytest

import inputs
from tests.gpu_util import assert_bits_equal, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def r9k():
    import torch
    import block_scaled_fp8_r9k_amd as m
    assert torch.cuda.is_available()
    m.lib()
    m.set_dispatch(255, m.ENGINE_AUTO)
    return m


def _p(t):
    return c_void_p(t.data_ptr())


def _noalloc(r9k, a, w, ws, c, packed):
    import torch
    M, K = a.shape
    N = w.shape[0]
    rc = r9k.lib().r9k_gemm_fp8_block_qa_noalloc(_p(a), M, K, _p(w), _p(ws), N, _p(c), 1 if packed else 0,
                                                 c_void_p(torch.cuda.current_stream().cuda_stream))
    return rc


def _reference(r9k, a, w, ws, packed):
    import torch
    M, K = a.shape
    N = w.shape[0]
    wsp = torch.zeros(r9k.gemm_fp8_block_workspace(M, K, N), dtype=torch.uint8, device="cuda")
    f = r9k.gemm_fp8_block_qa_packed if packed else r9k.gemm_fp8_block_qa
    return host(f(a, w, ws, workspace=wsp))


@pytest.mark.parametrize("packed", [False, True])
def test_noalloc_equals_workspace_entry(r9k, packed):
    import torch
    # first a mid-width call with a K split (quantised activations and fp32 partials in the scratch), then
    # a smaller mid-width call without one, then a smaller decode-width call with a K split (fp32 partials
    # in the scratch, over what the earlier calls left there)
    shapes = [(64, 14336, 4096), (32, 4096, 4096), (16, 14336, 2048)]
    for i, (M, K, N) in enumerate(shapes):
        say("noalloc", packed, M, K, N)
        a = dev(inputs.activations(40 + i, M, K, outliers=True))
        wq, ws = r9k.quant_weight(dev(inputs.weights(40 + i, N, K)))
        w = r9k.pack_weight(wq) if packed else wq
        want = _reference(r9k, a, w, ws, packed)
        c = torch.full((M, N), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        assert _noalloc(r9k, a, w, ws, c, packed) == 0
        torch.cuda.synchronize()
        assert_bits_equal(host(c), want, f"noalloc {M}x{K}x{N} packed={packed}")
        # the binding's wrapper gives the same bits
        assert_bits_equal(host(r9k.gemm_fp8_block_qa_noalloc(a, w, ws, packed=packed)), want, "binding")


def test_noalloc_limits_and_arguments(r9k):
    import torch
    a = torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((128, 128), dtype=torch.uint8, device="cuda")
    ws = torch.ones((1, 1), dtype=torch.float32, device="cuda")
    c = torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda")
    L = r9k.lib()
    s = c_void_p(None)
    assert L.r9k_gemm_fp8_block_qa_noalloc(_p(a), 8, 128, _p(w), _p(ws), 128, _p(c), 2, s) == -7
    assert L.r9k_gemm_fp8_block_qa_noalloc(c_void_p(None), 8, 128, _p(w), _p(ws), 128, _p(c), 0, s) == -1
    # a shape whose workspace exceeds the scratch is refused before any launch (the pointers are not read)
    big = 8192
    assert r9k.gemm_fp8_block_workspace(big, big, 1024) > r9k.NOALLOC_SCRATCH_BYTES
    assert L.r9k_gemm_fp8_block_qa_noalloc(_p(a), big, big, _p(w), _p(ws), 1024, _p(c), 0, s) == -6
