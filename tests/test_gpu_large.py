"""The dense GEMM at large and ragged sizes through the dispatcher, against the oracle.

Decode widths are compared in full; wide shapes on every column of a few rows (the first, second, middle and
last) plus random positions, with the RMS taken over those oracle values.  The shapes reach past the
workload's: a 28672 x 8192 weight (235 MB) streamed at 16 rows, K = 28672 at one row (the K split), an
8192-cube prefill, and ragged edges in both M and N (4097 rows, N = 33 x 128, a half-full last column tile).
Both weight layouts are checked against the oracle and against each other (equal up to the fp32 summation
order, where the decode planner slices K differently for them).
"""
import numpy as np
import pytest

import inputs
from tests.gpu_util import assert_close, assert_layouts_agree, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def r9k():
    import torch
    import block_scaled_fp8_r9k_amd as m
    assert torch.cuda.is_available()
    m.lib()
    m.set_dispatch(255, m.ENGINE_AUTO)
    return m


def _run(r9k, ora, M, K, N, seed):
    a = inputs.activations(seed, M, K, outliers=True)
    w = inputs.weights(seed + 1, N, K)
    wq_o, ws_o = ora.quant_weight(w)
    aq_o, as_o = ora.quant_act(a)
    a_d = dev(a)
    wq, ws = r9k.quant_weight(dev(w))
    del w
    got = host(r9k.gemm_fp8_block_qa(a_d, wq, ws))
    packed = host(r9k.gemm_fp8_block_qa_packed(a_d, r9k.pack_weight(wq), ws))
    assert_layouts_agree(ora, packed, got, f"packed vs row-major {M}x{K}x{N}")
    return got, packed, (aq_o, as_o, wq_o, ws_o)


@pytest.mark.parametrize("M,K,N", [(16, 8192, 28672), (1, 28672, 8192), (5, 8192, 4224)])
def test_decode_widths_large(r9k, ora, M, K, N):
    say("large decode", M, K, N)
    got, packed, (aq, as_, wq, ws) = _run(r9k, ora, M, K, N, seed=M + K // 128)
    _, c64 = ora.gemm_block(aq, as_, wq, ws, want_f64=True)
    assert_close(ora, got, c64, f"large decode {M}x{K}x{N}")
    assert_close(ora, packed, c64, f"large decode, packed {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N", [(8192, 8192, 8192), (4097, 4096, 4224), (300, 14336, 28672)])
def test_wide_large_sampled(r9k, ora, M, K, N):
    say("large wide", M, K, N)
    got, packed, (aq, as_, wq, ws) = _run(r9k, ora, M, K, N, seed=M % 1000 + K // 128)
    rows = np.unique(np.array([0, 1, M // 2, M - 1]))
    r = np.random.default_rng(M + N)
    ms = np.concatenate([np.repeat(rows, N), r.integers(0, M, 6000)])
    ns = np.concatenate([np.tile(np.arange(N), len(rows)), r.integers(0, N, 6000)])
    _, c64 = ora.gemm_block_at(aq, as_, wq, ws, ms, ns, want_f64=True)
    assert_close(ora, got[ms, ns], c64, f"large wide {M}x{K}x{N}")
    assert_close(ora, packed[ms, ns], c64, f"large wide, packed {M}x{K}x{N}")
