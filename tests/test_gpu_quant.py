"""GPU parity: the e4m3 encoder and the activation / weight quant kernels,
bit-exact against the oracle (codes and fp32 scale bits)."""
import numpy as np
import pytest

import inputs
from tests.gpu_util import assert_bits_equal, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def r9k():
    import torch
    import block_scaled_fp8_r9k_amd as r9k
    assert torch.cuda.is_available()
    r9k.lib()
    return r9k


def test_encode_every_binary32(r9k, ora):
    """Every non-NaN binary32 pattern through the device encoder, against the oracle."""
    import torch
    chunk = 1 << 28
    for lo in range(0, 1 << 32, chunk):
        say(f"encode chunk {lo >> 28} of 16")
        pats = (np.arange(lo, lo + chunk, dtype=np.int64) & 0xFFFFFFFF).astype(np.uint32)
        x = pats.view(np.float32)
        xt = torch.from_numpy(x).cuda()
        got = host(r9k.encode_e4m3(xt))
        want = ora.e4m3_encode(x)
        keep = ~np.isnan(x)
        bad = np.nonzero((got != want) & keep)[0]
        assert bad.size == 0, (f"{bad.size} mismatches in chunk {lo >> 28}; first x={x[bad[0]]!r} "
                               f"bits={pats[bad[0]]:#010x} gpu={got[bad[0]]:#x} oracle={want[bad[0]]:#x}")
        del xt
    torch.cuda.synchronize()


def test_encode_tail_lengths(r9k, ora):
    import torch
    r = np.random.default_rng(0)
    for n in (1, 2, 3, 5, 7, 1023, 1025):
        x = (r.standard_normal(n) * 100).astype(np.float32)
        got = host(r9k.encode_e4m3(torch.from_numpy(x).cuda()))
        assert_bits_equal(got, ora.e4m3_encode(x), f"encode n={n}")


def _check_quant_act(r9k, ora, a_bits, what):
    say("quant_act", what, a_bits.shape)
    aq, as_ = r9k.quant_act(dev(a_bits))
    q_o, s_o = ora.quant_act(a_bits)
    assert_bits_equal(host(aq), q_o, what + " codes")
    assert_bits_equal(host(as_), s_o, what + " scales")


def test_quant_act_edge_groups(r9k, ora):
    _check_quant_act(r9k, ora, inputs.quant_edge_groups(), "edge groups")


def test_quant_act_near_ties(r9k, ora):
    from tests.test_oracle_quant import _near_tie_rows
    _check_quant_act(r9k, ora, _near_tie_rows(5, 2000).reshape(50, -1), "near-tie groups")


@pytest.mark.parametrize("M,K", [(1, 512), (16, 4096), (255, 14336), (4096, 4096), (3, 128), (513, 16512)])
def test_quant_act_workloads(r9k, ora, M, K):
    _check_quant_act(r9k, ora, inputs.activations(0, M, K, outliers=K > 512), f"workload {M}x{K}")


def test_quant_act_every_amax(r9k, ora):
    """One group per positive finite bf16 amax (and amax = 0): the maximum at a
    rotating position, 127 other values of random sign and magnitude below it."""
    r = np.random.default_rng(11)
    amax = np.arange(0, 0x7F80, dtype=np.uint32)                 # 0 .. largest finite bf16
    G = amax.size
    lo = r.integers(0, amax[:, None] + 1, (G, 127), dtype=np.uint32)
    sign = (r.integers(0, 2, (G, 127), dtype=np.uint32) << 15)
    grp = np.concatenate([amax[:, None], lo | sign], axis=1)
    pos = np.arange(G) % 128                                      # move the maximum around
    rows = np.arange(G)
    grp[rows, 0], grp[rows, pos] = grp[rows, pos], grp[rows, 0].copy()
    assert G % 32 == 0
    _check_quant_act(r9k, ora, grp.astype(np.uint16).reshape(-1, 128 * 32), "every amax")


@pytest.mark.parametrize("N,K", [(1024, 512), (14336, 4096), (256, 128)])
def test_quant_weight(r9k, ora, N, K):
    w = inputs.weights(0, N, K)
    if N == 256:
        w[128:, :] = 0                                           # an all-zero block
        w[0, 0] = 0x7F7F                                         # largest finite bf16
    say("quant_weight", N, K)
    wq, ws = r9k.quant_weight(dev(w))
    q_o, s_o = ora.quant_weight(w)
    assert_bits_equal(host(wq), q_o, f"weight codes {N}x{K}")
    assert_bits_equal(host(ws), s_o, f"weight scales {N}x{K}")
