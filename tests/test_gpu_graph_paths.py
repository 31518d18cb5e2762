"""The routing, the MoE decode with a shared expert's term and the bf16-activation GEMM captured in one
HIP graph: every replay must give the eager calls' bits, with eager work on the same buffers between
the replays."""
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


def test_route_moe_bf16a_in_hip_graph(r9k):
    import torch
    T, H, E, I, k = 8, 1024, 16, 256, 4
    x, logits, w13, w2 = inputs.moe_inputs(21, T, H, E, I)
    w13q, w13s = r9k.quant_weight(dev(w13.reshape(E * 2 * I, H)))
    w2q, w2s = r9k.quant_weight(dev(w2.reshape(E * H, I)))
    w13p = r9k.pack_weight(w13q).view(E, 2 * I, H)
    w2p = r9k.pack_weight(w2q).view(E, H, I)
    w13s, w2s = w13s.view(E, 2 * I // 128, H // 128), w2s.view(E, H // 128, I // 128)
    x_d, lg_d = dev(x), torch.from_numpy(logits).cuda()
    r = np.random.default_rng(22)
    s_d = dev(inputs.to_bf16_bits(r.standard_normal((T, H)).astype(np.float32)))
    g_d = torch.from_numpy(r.random(T).astype(np.float32)).cuda()
    M, K, N = 4, 2048, 4096
    a_d = dev(inputs.activations(23, M, K, outliers=True))
    wq, ws = r9k.quant_weight(dev(inputs.weights(24, N, K)))
    wp = r9k.pack_weight(wq)

    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, k), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mws = torch.zeros(r9k.moe_fp8_decode_workspace(T, H, E, I, k), dtype=torch.uint8, device="cuda")

    def calls(stream=None):
        r9k.moe_route(lg_d, k, ids=ids, w=wts, stream=stream)
        r9k.moe_fp8_decode(x_d, ids, wts, w13p, w13s, w2p, w2s, out=out, workspace=mws, fused=True,
                           packed=True, shared=s_d, shared_w=g_d, stream=stream)
        r9k.gemm_fp8_block_bf16a(a_d, wp, ws, c=c, packed=True, stream=stream)

    calls()
    torch.cuda.synchronize()
    eager = [host(t) for t in (ids, wts, out, c)]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            calls(stream=s)
    torch.cuda.current_stream().wait_stream(s)
    names = ("route ids", "route weights", "moe out", "bf16a out")
    for rep in range(4):
        say("graph paths replay", rep)
        for t in (ids, wts, out, c):
            t.zero_()
        # eager work between replays: the three-launch MoE path over the same workspace
        r9k.moe_fp8_decode(x_d, ids, wts, w13p, w13s, w2p, w2s, workspace=mws, fused=False, packed=True)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e, name in zip((ids, wts, out, c), eager, names):
            assert_bits_equal(host(t), e, f"graph {name} replay {rep}")
