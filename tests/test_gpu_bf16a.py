"""The bf16-activation variant (fp8 block weights against unquantised bf16 activations, decode widths)
against the oracle, through the C ABI, on both weight layouts."""
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
    return m


def _check(ora, got, want64, what):
    """Within one bf16 ulp of the binary64 value plus fp32 accumulation slack (1e-5 of the RMS): there is no
    activation quant, so this is much tighter than the quantised path's bar."""
    o = np.asarray(want64, np.float64)
    g = ora.bf16_value(got).astype(np.float64)
    rms = float(np.sqrt(np.mean(o * o))) if o.size else 0.0
    bound = ora.bf16_ulp(o) + 1e-5 * rms
    err = np.abs(g - o)
    assert np.all(err <= bound), f"{what}: worst {float(np.max(err / bound)):.3f} of the bound"


_W = {}


def _weights(ora, r9k, N, K, seed):
    key = (N, K, seed)
    if key not in _W:
        w = inputs.weights(seed, N, K)
        wq, ws = r9k.quant_weight(dev(w))
        _W.clear()
        _W[key] = (wq, ws, host(wq), host(ws), r9k.pack_weight(wq))
    return _W[key]


@pytest.mark.parametrize("M,K,N", [(1, 4096, 14336), (2, 4096, 14336), (4, 4096, 14336), (8, 4096, 14336),
                                   (16, 4096, 14336), (5, 14336, 4096), (16, 14336, 4096), (3, 7168, 1024),
                                   (1, 128, 128), (7, 384, 256), (13, 640, 384), (9, 1280, 512), (16, 2048, 2048),
                                   # long staged rows whose K/1024 does not divide sixteen (three slices)
                                   (16, 3072, 4096), (12, 3072, 4096), (16, 6144, 2048),
                                   # from 5 rows two tiles a CTA down to 168 CTAs
                                   (8, 2048, 6144), (6, 4096, 5376),
                                   # wide rows with few sixteen-wave CTAs: eight waves of half the tiles
                                   (9, 4096, 4096), (16, 8192, 2048)])
def test_bf16a_against_oracle(r9k, ora, M, K, N):
    say("bf16a", M, K, N)
    a = inputs.activations(M + K // 128, M, K, outliers=True)
    wq, ws, wq_h, ws_h, wp = _weights(ora, r9k, N, K, seed=K // 128)
    c = host(r9k.gemm_fp8_block_bf16a(dev(a), wq, ws))
    _, c64 = ora.gemm_block_bf16a(a, wq_h, ws_h, want_f64=True)
    _check(ora, c, c64, f"bf16a {M}x{K}x{N}")
    assert_bits_equal(host(r9k.gemm_fp8_block_bf16a(dev(a), wp, ws, packed=True)), c, "packed == row-major")
    assert_bits_equal(host(r9k.gemm_fp8_block_bf16a(dev(a), wq, ws)), c, "repeat")


def test_bf16a_edge_values(r9k, ora):
    """Zero rows, subnormal bf16 activations, the largest e4m3 weights and values of both signs."""
    M, K, N = 6, 1024, 256
    a = inputs.activations(70, M, K, outliers=True)
    a[1] = 0                                  # a zero row gives +0 everywhere
    a[2, ::3] = 0x0001                        # smallest subnormal bf16
    a[3] = inputs.to_bf16_bits(np.full(K, -1e30, np.float32))
    wq, ws, wq_h, ws_h, wp = _weights(ora, r9k, N, K, seed=71)
    c = host(r9k.gemm_fp8_block_bf16a(dev(a), wq, ws))
    _, c64 = ora.gemm_block_bf16a(a, wq_h, ws_h, want_f64=True)
    for m in range(M):  # each row against its own scale (row 3 is 1e30 times the others)
        if m != 1:
            _check(ora, c[m:m + 1], c64[m:m + 1], f"bf16a edge values, row {m}")
    assert np.all(c[1] == 0)


def test_bf16a_shape_errors(r9k):
    import torch
    a = torch.zeros((17, 1024), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((256, 1024), dtype=torch.uint8, device="cuda")
    ws = torch.zeros((2, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(r9k.R9kError) as e:
        r9k.gemm_fp8_block_bf16a(a, w, ws)                      # M > 16
    assert e.value.code == -2
    a = torch.zeros((1, 128 * 17), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((256, 128 * 17), dtype=torch.uint8, device="cuda")
    ws = torch.zeros((2, 17), dtype=torch.float32, device="cuda")
    with pytest.raises(r9k.R9kError) as e:
        r9k.gemm_fp8_block_bf16a(a, w, ws)                      # K/128 = 17 has no launch shape
    assert e.value.code == -2
    # M = 0 with valid pointers launches nothing and succeeds (a null pointer is an error whatever M is)
    from ctypes import c_void_p
    a = torch.zeros((1, 1024), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((256, 1024), dtype=torch.uint8, device="cuda")
    ws = torch.zeros((2, 8), dtype=torch.float32, device="cuda")
    c = torch.full((1, 256), 7, dtype=torch.int16, device="cuda")
    rc = r9k.lib().r9k_gemm_fp8_block_bf16a(c_void_p(a.data_ptr()), 0, 1024, c_void_p(w.data_ptr()),
                                            c_void_p(ws.data_ptr()), 256, c_void_p(c.data_ptr()), c_void_p(None))
    torch.cuda.synchronize()
    assert rc == 0 and bool(torch.all(c == 7))
