"""GPU parity for the dense block-scaled GEMM through the C ABI.

Outputs must satisfy |gpu - oracle| <= 1e-2 * RMS(oracle) + 1 bf16 ulp(oracle)
elementwise (RMS over the whole output of the call; for sampled checks, over
the sampled oracle values).  The fused form must equal the split form bit for
bit, both engines must pass at every M (forced), and repeated runs must be
bitwise identical.
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


class Problem:
    """Seeded inputs; the GPU quantises the weights with its own kernel and
    the oracle with its own code (the quant parity is tested separately)."""

    def __init__(self, r9k, ora, M, K, N, seed=0, outliers=True):
        self.M, self.K, self.N = M, K, N
        self.a = inputs.activations(seed, M, K, outliers=outliers)
        self.w = inputs.weights(seed, N, K)
        self.wq_o, self.ws_o = ora.quant_weight(self.w)
        self.aq_o, self.as_o = ora.quant_act(self.a)
        self.a_d = dev(self.a)
        self.wq_d, self.ws_d = r9k.quant_weight(dev(self.w))

    def oracle_full(self, ora):
        _, c64 = ora.gemm_block(self.aq_o, self.as_o, self.wq_o, self.ws_o, want_f64=True)
        return c64

    def run(self, r9k, engine, fused=True):
        r9k.set_dispatch(255, engine)
        if fused:
            return host(r9k.gemm_fp8_block_qa(self.a_d, self.wq_d, self.ws_d))
        aq, as_ = r9k.quant_act(self.a_d)
        return host(r9k.gemm_fp8_block(aq, as_, self.wq_d, self.ws_d))


ENGINES = {"skinny": 1, "tiled": 2}


@pytest.mark.parametrize("M,K,N", [(1, 512, 1024), (1, 128, 128), (3, 384, 256), (16, 1024, 384),
                                   (17, 256, 640), (33, 640, 256), (100, 384, 384), (255, 512, 256),
                                   (256, 512, 256), (300, 256, 384), (129, 1280, 128)])
@pytest.mark.parametrize("engine", ["skinny", "tiled"])
def test_gemm_small_shapes(r9k, ora, M, K, N, engine):
    say("gemm", engine, M, K, N)
    p = Problem(r9k, ora, M, K, N, seed=M * 7 + K)
    c64 = p.oracle_full(ora)
    fused = p.run(r9k, ENGINES[engine], fused=True)
    assert_close(ora, fused, c64, f"{engine} fused {M}x{K}x{N}")
    split = p.run(r9k, ENGINES[engine], fused=False)
    assert_bits_equal(fused, split, f"{engine} fused vs split {M}x{K}x{N}")
    again = p.run(r9k, ENGINES[engine], fused=True)
    assert_bits_equal(fused, again, f"{engine} repeat {M}x{K}x{N}")


@pytest.mark.parametrize("M", [1, 2, 4, 8, 9, 10, 11, 16])
def test_gemm_decode_sweep_full(r9k, ora, M):
    """M in {1,2,4,8,16} and the odd widths 9-11 (the first rows of the wide
    CTAs), K=4096, N=14336, every output against the oracle."""
    say("decode sweep", M)
    p = Problem(r9k, ora, M, 4096, 14336)
    c64 = p.oracle_full(ora)
    got = p.run(r9k, 0, fused=True)
    assert_close(ora, got, c64, f"decode M={M}")
    assert_bits_equal(got, p.run(r9k, 0, fused=False), f"decode M={M} fused vs split")


def _sampled(ora, p, rows, n_random=4000, seed=3):
    r = np.random.default_rng(seed)
    ms = np.concatenate([np.repeat(rows, p.N), r.integers(0, p.M, n_random)])
    ns = np.concatenate([np.tile(np.arange(p.N), len(rows)), r.integers(0, p.N, n_random)])
    _, c64 = ora.gemm_block_at(p.aq_o, p.as_o, p.wq_o, p.ws_o, ms, ns, want_f64=True)
    return ms, ns, c64


@pytest.mark.parametrize("M,K", [(32, 4096), (64, 4096), (128, 14336), (255, 4096), (255, 14336)])
def test_gemm_mid_sweep_sampled(r9k, ora, M, K):
    say("mid sweep", M, K)
    p = Problem(r9k, ora, M, K, 4096)
    rows = np.unique(np.array([0, 1, M // 2, M - 1]))
    ms, ns, c64 = _sampled(ora, p, rows)
    got = p.run(r9k, 0, fused=True)
    assert_close(ora, got[ms, ns], c64, f"mid M={M} K={K}")
    assert_bits_equal(got, p.run(r9k, 0, fused=False), f"mid M={M} fused vs split")


@pytest.mark.parametrize("M,K,N", [(65, 4096, 14336), (255, 4096, 14336), (129, 4096, 6144), (65, 14336, 4096),
                                   (100, 8192, 4096)])
def test_gemm_wide_mid_rows_go_tiled(r9k, ora, M, K, N):
    """65 to 255 rows where the tiled engine is the automatic choice (long K, or the mid-width kernel's
    64 x 64 blocks more than one CTA per compute unit): sampled rows and points against the oracle,
    and the fused call equal to the split call."""
    for packed in (False, True):
        assert r9k.gemm_fp8_block_plan(M, K, N, packed)[0] == r9k.KERNEL_TILED
    say("wide mid rows", M, K, N)
    p = Problem(r9k, ora, M, K, N, seed=11)
    rows = np.unique(np.array([0, 1, M // 2, M - 1]))
    ms, ns, c64 = _sampled(ora, p, rows)
    got = p.run(r9k, 0, fused=True)
    assert_close(ora, got[ms, ns], c64, f"tiled route {M}x{K}x{N}")
    assert_bits_equal(got, p.run(r9k, 0, fused=False), f"tiled route {M}x{K}x{N} fused vs split")


def test_gemm_boundary_both_engines(r9k, ora):
    """M = 255 and 256 at K=4096, N=4096, each engine forced."""
    for M in (255, 256):
        p = Problem(r9k, ora, M, 4096, 4096, seed=M)
        rows = np.array([0, 127, 128, M - 1])
        ms, ns, c64 = _sampled(ora, p, rows)
        outs = {}
        for name, e in ENGINES.items():
            say("boundary", M, name)
            outs[name] = p.run(r9k, e, fused=True)
            assert_close(ora, outs[name][ms, ns], c64, f"boundary M={M} {name}")


def test_gemm_prefill_sampled(r9k, ora):
    """M=4096, K=4096, N=12288 (the prefill chunk), auto dispatch, sampled outputs."""
    say("prefill 4096x4096x12288")
    p = Problem(r9k, ora, 4096, 4096, 12288)
    rows = np.array([0, 1, 127, 128, 2047, 4095])
    ms, ns, c64 = _sampled(ora, p, rows, n_random=20000)
    got = p.run(r9k, 0, fused=True)
    assert_close(ora, got[ms, ns], c64, "prefill")
    again = p.run(r9k, 0, fused=True)
    assert_bits_equal(got, again, "prefill repeat")


def test_gemm_reuses_workspace_and_streams(r9k, ora):
    """Two shapes in a row through one explicit workspace, on a side stream:
    each call writes what it reads, so reuse gives the same results."""
    import torch
    p1 = Problem(r9k, ora, 8, 4096, 2048, seed=5)
    p2 = Problem(r9k, ora, 3, 1024, 1024, seed=6)
    nbytes = max(r9k.gemm_fp8_block_workspace(8, 4096, 2048), r9k.gemm_fp8_block_workspace(3, 1024, 1024))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    r9k.set_dispatch(255, 0)
    outs = []
    with torch.cuda.stream(s):
        for p in (p1, p2, p1, p2):
            outs.append(r9k.gemm_fp8_block_qa(p.a_d, p.wq_d, p.ws_d, workspace=ws, stream=s))
    s.synchronize()
    assert_close(ora, host(outs[0]), p1.oracle_full(ora), "stream p1")
    assert_close(ora, host(outs[1]), p2.oracle_full(ora), "stream p2")
    assert_bits_equal(host(outs[0]), host(outs[2]), "p1 twice")
    assert_bits_equal(host(outs[1]), host(outs[3]), "p2 twice")


def test_binding_takes_the_current_stream(r9k, ora):
    """With no stream argument the binding launches on torch's current stream
    (read as a raw handle): the default stream, then a side stream entered with
    torch.cuda.stream; the call made there is correct once that stream is done."""
    import torch
    handle = lambda: r9k._stream(None).value or 0  # ctypes reads the null handle (the default stream) as None
    assert handle() == torch.cuda.current_stream().cuda_stream
    p = Problem(r9k, ora, 4, 1024, 1024, seed=7)
    r9k.set_dispatch(255, 0)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert handle() == s.cuda_stream
        out = r9k.gemm_fp8_block_qa(p.a_d, p.wq_d, p.ws_d)
    s.synchronize()
    assert_close(ora, host(out), p.oracle_full(ora), "current side stream")


def test_gemm_in_hip_graph(r9k, ora):
    """Captured calls of every route replay to the eager result, several times, with eager calls on the
    same workspaces between the replays: decode, decode with a K split (partials + reduce launch), the
    mid-width kernel (quant launch + GEMM) with and without its K split, and prefill (tiled)."""
    import torch
    r9k.set_dispatch(255, 0)
    shapes = [(4, 4096, 4096), (16, 14336, 2048), (64, 4096, 4096), (32, 14336, 4096), (512, 1024, 1024)]
    probs = [Problem(r9k, ora, M, K, N, seed=8 + i) for i, (M, K, N) in enumerate(shapes)]
    wss = [torch.zeros(r9k.gemm_fp8_block_workspace(M, K, N), dtype=torch.uint8, device="cuda")
           for M, K, N in shapes]
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for M, K, N in shapes]
    eager = [host(r9k.gemm_fp8_block_qa(p.a_d, p.wq_d, p.ws_d, workspace=w)) for p, w in zip(probs, wss)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for p, w, c in zip(probs, wss, outs):
                r9k.gemm_fp8_block_qa(p.a_d, p.wq_d, p.ws_d, c=c, workspace=w)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        say("graph replay", rep)
        for c in outs:
            c.zero_()
        # eager work on the same workspaces: each call of the next shape's problem is run on this one's
        # workspace where it fits, leaving other contents there
        for k, (p, w) in enumerate(zip(probs, wss)):
            q = probs[(k + 1) % len(probs)]
            if w.numel() >= r9k.gemm_fp8_block_workspace(q.M, q.K, q.N):
                r9k.gemm_fp8_block_qa(q.a_d, q.wq_d, q.ws_d, workspace=w)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (M, K, N), c, e in zip(shapes, outs, eager):
            assert_bits_equal(host(c), e, f"graph {M}x{K}x{N} replay {rep}")


@pytest.mark.parametrize("M,K,N", [(17, 4096, 14336), (24, 1024, 4096), (20, 1536, 3072), (24, 2048, 8192),
                                   (24, 2048, 14336), (6, 14336, 1024)])
def test_gemm_decode_two_row_tiles(r9k, ora, M, K, N):
    """The decode kernel's widths past 16 rows (two row tiles) and K=14336 at 6 rows, full output, both
    weight layouts (which may slice K differently: equal up to the fp32 summation order)."""
    say("decode widths", M, K, N)
    for packed in (False, True):
        assert r9k.gemm_fp8_block_plan(M, K, N, packed) == (r9k.KERNEL_DECODE, 1), (M, K, N, packed)
    p = Problem(r9k, ora, M, K, N, seed=M + 3)
    c64 = p.oracle_full(ora)
    got = p.run(r9k, 0, fused=True)
    assert_close(ora, got, c64, f"decode {M}x{K}x{N}")
    wp = r9k.pack_weight(p.wq_d)
    assert_layouts_agree(ora, host(r9k.gemm_fp8_block_qa_packed(p.a_d, wp, p.ws_d)), got, "packed vs row-major")
    assert_bits_equal(p.run(r9k, 0, fused=False), got, "split == fused")


@pytest.mark.parametrize("M,K,N", [(16, 14336, 4096), (8, 14336, 4096), (16, 14336, 2048), (12, 14336, 2048),
                                   (1, 28672, 1024)])
def test_gemm_decode_k_split(r9k, ora, M, K, N):
    """Decode-kernel shapes that split K across CTAs (fp32 partials + ordered reduce), full output,
    both weight layouts (equal up to the fp32 summation order), fused == split form."""
    for packed in (False, True):
        kern, ks = r9k.gemm_fp8_block_plan(M, K, N, packed)
        assert kern == r9k.KERNEL_DECODE and ks > 1, (packed, kern, ks)
    say("decode k-split", M, K, N)
    p = Problem(r9k, ora, M, K, N, seed=M + 11)
    c64 = p.oracle_full(ora)
    got = p.run(r9k, 0, fused=True)
    assert_close(ora, got, c64, f"decode k-split {M}x{K}x{N}")
    wp = r9k.pack_weight(p.wq_d)
    assert_layouts_agree(ora, host(r9k.gemm_fp8_block_qa_packed(p.a_d, wp, p.ws_d)), got, "packed vs row-major")
    assert_bits_equal(p.run(r9k, 0, fused=False), got, "split == fused")
    assert_bits_equal(p.run(r9k, 0, fused=True), got, "repeat")


def test_gemm_wide_n_skinny_inload_quant(r9k, ora):
    """A wide output at a decode width (16 rows of an 8192 -> 32768 projection) on the split-K skinny
    kernel (forced: the dispatcher gives this shape to the mid-width kernel) with the activation quant in
    its A-load and a K split: sampled outputs against the oracle, fused == split bit for bit, both weight
    layouts."""
    M, K, N = 16, 8192, 32768
    assert r9k.gemm_fp8_block_plan(M, K, N)[0] == r9k.KERNEL_MID
    r9k.set_dispatch(255, r9k.ENGINE_SPLITK)
    try:
        _wide_n_skinny(r9k, ora, M, K, N)
    finally:
        r9k.set_dispatch(255, r9k.ENGINE_AUTO)


def _wide_n_skinny(r9k, ora, M, K, N):
    for packed in (False, True):
        assert r9k.gemm_fp8_block_plan(M, K, N, packed)[0] == r9k.KERNEL_SKINNY
    say("wide-N skinny", M, K, N)
    p = Problem(r9k, ora, M, K, N, seed=21)
    rows = np.array([0, 1, 7, 15])
    ms, ns, c64 = _sampled(ora, p, rows, n_random=8000)
    got = p.run(r9k, 0, fused=True)
    assert_close(ora, got[ms, ns], c64, "wide-N skinny")
    assert_bits_equal(got, p.run(r9k, 0, fused=False), "wide-N skinny fused vs split")
    wp = r9k.pack_weight(p.wq_d)
    assert_bits_equal(host(r9k.gemm_fp8_block_qa_packed(p.a_d, wp, p.ws_d)), got, "wide-N skinny packed")


def test_gemm_lm_head_width_decode(r9k, ora):
    """An LM-head-wide output at decode widths (8 rows of a 4096 -> 65536 projection) on the decode kernel
    over all of K: sampled outputs against the oracle on both weight layouts (which may slice K
    differently, so each is checked on its own), fused == split bit for bit."""
    M, K, N = 8, 4096, 65536
    for packed in (False, True):
        assert r9k.gemm_fp8_block_plan(M, K, N, packed) == (r9k.KERNEL_DECODE, 1)
    say("lm-head width decode", M, K, N)
    p = Problem(r9k, ora, M, K, N, seed=23)
    ms, ns, c64 = _sampled(ora, p, np.arange(M), n_random=4000)
    got = p.run(r9k, 0, fused=True)
    assert_close(ora, got[ms, ns], c64, "lm-head width decode")
    assert_bits_equal(got, p.run(r9k, 0, fused=False), "lm-head width decode fused vs split")
    wp = r9k.pack_weight(p.wq_d)
    gotp = host(r9k.gemm_fp8_block_qa_packed(p.a_d, wp, p.ws_d))
    assert_close(ora, gotp[ms, ns], c64, "lm-head width decode packed")


def test_gemm_empty_batch(r9k):
    """M = 0 through the binding returns an empty output without a launch, for every GEMM form."""
    import torch
    a = torch.empty((0, 4096), dtype=torch.bfloat16, device="cuda")
    aq = torch.empty((0, 4096), dtype=torch.uint8, device="cuda")
    as_ = torch.empty((0, 32), dtype=torch.float32, device="cuda")
    w = torch.zeros((4096, 4096), dtype=torch.uint8, device="cuda")
    ws = torch.ones((32, 32), dtype=torch.float32, device="cuda")
    for c in (r9k.gemm_fp8_block_qa(a, w, ws), r9k.gemm_fp8_block(aq, as_, w, ws),
              r9k.gemm_fp8_block_qa_packed(a, w, ws), r9k.gemm_fp8_block_packed(aq, as_, w, ws)):
        assert tuple(c.shape) == (0, 4096)
    assert r9k.gemm_fp8_block_workspace(0, 4096, 4096) == 0
    torch.cuda.synchronize()
