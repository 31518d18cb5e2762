#!/usr/bin/env python3
"""Benchmark of the block-scaled fp8 GEMM path on one MI355X.

Headline (one JSON line on stdout): the decode-width sweep, M in {1,2,4,8,16},
K=4096, N=14336, bf16 activations quantised per token in groups of 128 inside
the GEMM (r9k_gemm_fp8_block_qa), fp8 e4m3 weights with 128x128 fp32 block
scales, bf16 out.  One step = the five fused GEMM calls on one batch of
synthetic input; `value` is the algorithmic HBM bytes of the step divided by
its time (GB/s).  Inputs are resident in HBM before timing; the weights rotate
through enough distinct copies (>= 512 MB) that the 256 MB Infinity Cache
cannot hold them between launches: every launch, also within a step, reads a
copy that the previous launches did not.  Timing: HIP graphs replayed on the
current stream, bracketed by HIP events; one graph holds as many consecutive
steps as there are copies.

The same line carries:
  roofline      the dominant kernel (k_gemm_decode, the weight-streaming
                kernel of the decode widths): algorithmic bytes per launch /
                its average launch time vs 8 TB/s, averaged over the sweep;
                `traffic` is the HBM bytes per launch that the committed
                rocprofv3 counter summary measured on the same kernel source;
                `frac_of_read_ceiling` the same against hbm_read_ceiling;
  hbm_read_ceiling  a plain read (no compute) of the weight's byte count,
                timed like the decode launches: what this GPU streams at best;
  cpu_baseline  the CPU oracle timed on one full step of the same inputs;
  prefill       M=4096, K=4096, N=12288: fp8 TFLOP/s vs 5.03 PFLOP/s dense, for
                the fused call and (its `roofline`) for the GEMM kernel on
                codes quantised beforehand;
  mid           M in {32,64,128,255} at (K,N) = (4096,4096) and (14336,4096);
  moe           16 tokens, hidden 2048, 128 experts of 768, top-8: GB/s over
                the bytes of the experts the routing touches, plus the
                routing kernel and the fused path with a shared expert;
  single_token  M=1, K=512, N=1024 (seed 0, no outliers): microseconds a call;
  bf16a         the decode sweep on the bf16-activation variant (no quant).
Every leg's GPU time is the median of TRIALS (5) timed trials, each over many
launches, with the trials listed; prefill, mid, moe and single_token each carry
a `cpu_baseline` of their own (the oracle on the leg's workload, or a stated
sample of it, median of up to 3 runs).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--only decode,prefill,mid,moe,single_token,bf16a] [--mid-points 255x4096,...]
                       [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5033.2        # 256 CU x 2.4 GHz x 8192 flop/CU/clk, dense fp8 MFMA
DECODE_M = (1, 2, 4, 8, 16)
DECODE_K, DECODE_N = 4096, 14336
ROTATE_BYTES = 512 << 20
TRIALS = 5


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def gemm_bytes(M, K, N):
    """Algorithmic HBM bytes of one GEMM call: weight codes + block scales +
    bf16 activations read once + bf16 output."""
    return N * K + 4 * (N // 128) * (K // 128) + 2 * M * K + 2 * M * N


class Timer:
    def __init__(self, torch):
        self.torch = torch

    def run(self, fn, reps):
        torch = self.torch
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        for i in range(reps):
            fn(i)
        e.record()
        e.synchronize()
        return s.elapsed_time(e) / reps  # ms


def warm_graph(tm, g):
    """Replays of one graph alone for GRAPH_WARM_S before its timed trials: right after a heavy phase
    (the decode step loop) the next launches run about 5% slow for several milliseconds, which the kernel
    trace of the same run does not show and a couple of replays did not cover."""
    t_end = time.perf_counter() + GRAPH_WARM_S
    while time.perf_counter() < t_end:
        tm.run(lambda i: g.replay(), 2)


def median_of_trials(run_once, n=TRIALS):
    """Median of n timed trials (run_once() -> ms) and the trials themselves."""
    t = [run_once() for _ in range(n)]
    return float(np.median(t)), t


def cpu_seconds(fn, budget_s=10.0, max_runs=3):
    """Median wall time of up to max_runs calls of fn, stopping once budget_s is spent."""
    times = []
    while len(times) < max_runs and sum(times) < budget_s:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return float(np.median(times)), len(times)


def capture(torch, calls):
    """One HIP graph holding the given launches, captured on a side stream."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for c in calls:
                c()
    torch.cuda.current_stream().wait_stream(s)
    return g


def weight_copies(torch, r9k, dev, w_bits, min_bytes=ROTATE_BYTES, cap=40):
    """Quantise W once on the GPU (r9k_quant_weight) and make enough distinct
    device copies that rotating through them defeats the Infinity Cache."""
    wq, ws = r9k.quant_weight(dev(w_bits))
    n = max(2, min(cap, -(-min_bytes // wq.numel())))
    copies = [(wq, ws)] + [(wq.clone(), ws.clone()) for _ in range(n - 1)]
    torch.cuda.synchronize()
    return copies


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "k_gemm_decode_packed_sweep_k4096_n14336_traffic.md")
PREFILL_COUNTERS = os.path.join(ROOT, "profiles", "k_gemm_tiled_prefill_m4096_k4096_n12288_counters.md")
MID_COUNTERS = os.path.join(ROOT, "profiles", "k_gemm_mid_m255_k4096_n4096_counters.md")


def kernel_source_hash(kernel_file="gemm_decode.hip"):
    """Hash of the sources that make up one kernel (the decode kernel by
    default; a tuple names several kernel files) and its launch."""
    h = hashlib.sha256()
    files = (kernel_file,) if isinstance(kernel_file, str) else tuple(kernel_file)
    for f in files + ("r9k_device.h", "r9k_internal.h", "api.hip"):
        with open(os.path.join(ROOT, "block_scaled_fp8_r9k_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(summary=None, kernel_file="gemm_decode.hip"):
    """HBM bytes per launch of a kernel (the decode kernel over the sweep by
    default), from its committed rocprofv3 counter summary (lines
    `source_hash: ...` and `hbm_bytes_per_launch: ...`), if it was taken on
    the current source."""
    fields = {}
    try:
        with open(summary or TRAFFIC_SUMMARY) as fh:
            for ln in fh:
                k, sep, v = ln.partition(":")
                if sep and k.strip() in ("source_hash", "hbm_bytes_per_launch"):
                    fields[k.strip()] = v.strip().strip("`")
    except OSError:
        return None
    if fields.get("source_hash") != kernel_source_hash(kernel_file):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# --------------------------------------------------------------------------

def step_copy(c, j, n_per_step, n_copies):
    """The weight copy that launch j of step c reads: the launches of a step and the
    steps in turn walk the copies, so that a copy comes back only after n_copies
    launches (n_copies * |W| >= 512 MB, twice the Infinity Cache)."""
    return (c * n_per_step + j) % n_copies


def bench_decode(torch, r9k, inputs, dev, steps, warmup, packed=True):
    """The decode sweep.  packed: the weights in fragment order (r9k_pack_weight,
    done once at load like the quantisation, not timed); else row-major."""
    K, N = DECODE_K, DECODE_N
    Mmax = max(DECODE_M)
    a_bits = inputs.activations(0, Mmax, K, outliers=True)
    w_bits = inputs.weights(0, N, K)
    a = dev(a_bits)
    copies = weight_copies(torch, r9k, dev, w_bits)
    if packed:
        copies = [(r9k.pack_weight(wq), ws) for wq, ws in copies]
        torch.cuda.synchronize()
    gemm = r9k.gemm_fp8_block_qa_packed if packed else r9k.gemm_fp8_block_qa
    C = len(copies)
    log(f"decode ({'packed' if packed else 'row-major'} weights): {C} weight copies of "
        f"{copies[0][0].numel() / 1e6:.1f} MB")
    ws_bytes = max(r9k.gemm_fp8_block_workspace(M, K, N) for M in DECODE_M)
    wsp = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    outs = {M: torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for M in DECODE_M}
    a_rows = {M: a[:M].contiguous() for M in DECODE_M}

    def call(M, c):
        wq, ws = copies[c]
        return lambda: gemm(a_rows[M], wq, ws, c=outs[M], workspace=wsp)

    for c in range(C):  # eager warm-up of every call
        for M in DECODE_M:
            call(M, c)()
    torch.cuda.synchronize()
    # Every launch of a step reads its own weight copy (the step's five launches and the
    # steps in turn walk the copies), so that no launch finds its weights in the Infinity
    # Cache.  One graph holds C consecutive steps, as a decode step's many GEMMs sit in one
    # graph; `steps` not a multiple of C ends on single-step graphs.
    nM = len(DECODE_M)
    step_calls = [[call(M, step_copy(c, j, nM, C)) for j, M in enumerate(DECODE_M)] for c in range(C)]
    block_graph = capture(torch, [f for c in range(C) for f in step_calls[c]])
    step_graphs = [capture(torch, step_calls[c]) for c in range(C)]
    step_bytes = sum(gemm_bytes(M, K, N) for M in DECODE_M)
    tm = Timer(torch)

    def run_steps(n):  # exactly n steps: n // C block replays, then single steps
        def one(i):
            if i < n // C:
                block_graph.replay()
            else:
                step_graphs[i % C].replay()
        return one, n // C + n % C

    fn, calls = run_steps(max(warmup, 1))
    tm.run(fn, calls)
    fn, calls = run_steps(steps)
    ms_step = tm.run(fn, calls) * calls / steps

    # the dominant kernel alone: graphs of back-to-back launches at one M
    per_m = {}
    for M in DECODE_M:
        reps_per_graph = 2 * C
        g = capture(torch, [call(M, i % C) for i in range(reps_per_graph)])
        warm_graph(tm, g)
        ms, tr = median_of_trials(lambda: tm.run(lambda i: g.replay(), max(3, steps // 4)) / reps_per_graph)
        b = gemm_bytes(M, K, N)
        per_m[M] = dict(us=ms * 1e3, GBs=b / (ms * 1e-3) / 1e9, trials_us=[t * 1e3 for t in tr])
        log(f"decode M={M}: {ms * 1e3:.2f} us/launch, {per_m[M]['GBs']:.0f} GB/s")
    del step_graphs, block_graph, copies
    torch.cuda.empty_cache()
    us_avg = float(np.mean([per_m[M]["us"] for M in DECODE_M]))
    bytes_avg = float(np.mean([gemm_bytes(M, K, N) for M in DECODE_M]))
    achieved = bytes_avg / (us_avg * 1e-6) / 1e9
    return dict(ms_step=ms_step, step_bytes=step_bytes, per_m=per_m, achieved=achieved, us_avg=us_avg,
                bytes_avg=bytes_avg, a_bits=a_bits, w_bits=w_bits)


def bench_bf16a(torch, r9k, inputs, dev, reps):
    """The bf16-activation variant over the decode sweep (fragment-order weights, rotated as for the
    headline): per-launch time and GB/s of the same algorithmic bytes."""
    K, N = DECODE_K, DECODE_N
    a = dev(inputs.activations(0, max(DECODE_M), K, outliers=True))
    copies = weight_copies(torch, r9k, dev, inputs.weights(0, N, K))
    copies = [(r9k.pack_weight(wq), ws) for wq, ws in copies]
    C = len(copies)
    res = {}
    for M in DECODE_M:
        a_m = a[:M].contiguous()
        c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        calls = [lambda w=w, s=s: r9k.gemm_fp8_block_bf16a(a_m, w, s, c=c, packed=True) for w, s in copies] * 2
        for f in calls:
            f()
        g = capture(torch, calls)
        tm = Timer(torch)
        warm_graph(tm, g)
        ms, tr = median_of_trials(lambda: tm.run(lambda i: g.replay(), reps) / len(calls))
        res[str(M)] = dict(us=ms * 1e3, GBs=gemm_bytes(M, K, N) / (ms * 1e-3) / 1e9, trials_us=[t * 1e3 for t in tr])
        log(f"bf16a M={M}: {ms * 1e3:.2f} us/launch, {res[str(M)]['GBs']:.0f} GB/s")
    del copies
    torch.cuda.empty_cache()
    return dict(workload=f"M in {list(DECODE_M)}, K={K}, N={N}, bf16 activations (no quant), fragment-order "
                         f"weights", per_m=res)


def cpu_baseline(ora, a_bits, w_bits, step_bytes):
    """The oracle (exact fp64 group sums, one bf16 rounding) on one full step:
    activation quant + GEMM for every M of the sweep; weight quant is setup."""
    wq, ws = ora.quant_weight(w_bits)
    times = []
    t_total = 0.0
    while len(times) < 3 and t_total < 30.0:
        t0 = time.perf_counter()
        for M in DECODE_M:
            ora.gemm_block_qa(a_bits[:M], wq, ws)
        dt = time.perf_counter() - t0
        times.append(dt)
        t_total += dt
    t = float(np.median(times))
    return dict(value=step_bytes / t / 1e9, unit="GB/s", cores=ora.threads(), kind="oracle",
                seconds_per_step=t, repeats=len(times),
                sample=f"one full step: oracle group-128 act quant + exact block GEMM for M in "
                       f"{list(DECODE_M)}, K={DECODE_K}, N={DECODE_N} (weight quant not timed), "
                       f"median of {len(times)}")


GRAPH_WARM_S = 0.05  # seconds of one graph's replays before its timed trials (all legs but prefill)
PREFILL_WARM_S = 0.1  # seconds of alternating prefill launches before the timed trials


def bench_prefill(torch, r9k, inputs, dev, reps):
    M, K, N = 4096, 4096, 12288
    a = dev(inputs.activations(1, M, K, outliers=True))
    copies = weight_copies(torch, r9k, dev, inputs.weights(1, N, K))
    copies = [(r9k.pack_weight(wq), ws) for wq, ws in copies]  # fragment order, packed at load
    C = len(copies)
    wsp = torch.zeros(r9k.gemm_fp8_block_workspace(M, K, N), dtype=torch.uint8, device="cuda")
    c_out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    calls = [lambda c=c: r9k.gemm_fp8_block_qa_packed(a, copies[c][0], copies[c][1], c=c_out, workspace=wsp)
             for c in range(C)]
    # The GEMM kernel on its own: the split entry point on codes quantised once
    # beforehand is one k_gemm_tiled launch plus the transpose of the 4096 x 32
    # activation scales (a few microseconds), so this slightly understates the kernel.
    aq, as_ = r9k.quant_act(a)
    kcalls = [lambda c=c: r9k.gemm_fp8_block_packed(aq, as_, copies[c][0], copies[c][1], c=c_out, workspace=wsp)
              for c in range(C)]
    for f in calls + kcalls:
        f()
    g = capture(torch, calls)
    gk = capture(torch, kcalls)
    # Back-to-back prefill launches run 5-12% slower over their first 20-30 ms
    # on the MI355X (after the decode legs) and then hold within about 1%, so
    # both graphs first alternate for PREFILL_WARM_S; then each is timed over
    # `reps` back-to-back replays, TRIALS times, the two taking turns to go
    # first, and the median of each is taken.
    tm = Timer(torch)
    t_end = time.perf_counter() + PREFILL_WARM_S
    while time.perf_counter() < t_end:
        tm.run(lambda i: (g if i % 2 else gk).replay(), 2)
    tr, ktr = [], []
    for t in range(TRIALS):
        for leg in ((0, 1) if t % 2 == 0 else (1, 0)):
            if leg == 0:
                tr.append(tm.run(lambda i: g.replay(), reps) / C)
            else:
                ktr.append(tm.run(lambda i: gk.replay(), reps) / C)
    ms, kms = float(np.median(tr)), float(np.median(ktr))
    tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    ktf = 2.0 * M * N * K / (kms * 1e-3) / 1e12
    log(f"prefill {M}x{K}x{N}: {ms * 1e3:.1f} us, {tflops:.0f} TFLOP/s")
    log(f"prefill GEMM kernel (pre-quantised A): {kms * 1e3:.1f} us, {ktf:.0f} TFLOP/s")
    roof = dict(bound="mfma", achieved=ktf, peak=FP8_PEAK_TFLOPS, unit="TFLOP/s", frac=ktf / FP8_PEAK_TFLOPS,
                traffic=traffic_from_profiles(PREFILL_COUNTERS, "gemm_tiled.hip"),
                kernel="k_gemm_tiled (256 x 256 tile, fragment-order weights) with the scale transpose, per call",
                flops_per_launch=2.0 * M * N * K, us_per_launch=kms * 1e3)
    return dict(workload=f"M={M}, K={K}, N={N}, fused act quant, fragment-order weights", us=ms * 1e3,
                value=tflops, unit="TFLOP/s", peak=FP8_PEAK_TFLOPS, frac=tflops / FP8_PEAK_TFLOPS, roofline=roof,
                trials_us=[t * 1e3 for t in tr], codes_trials_us=[t * 1e3 for t in ktr],
                fused_over_codes=ms / kms)


KERNEL_NAMES = {1: "decode", 2: "skinny", 3: "tiled", 4: "mid"}


MID_POINTS = tuple((M, K) for K in (4096, 14336) for M in (32, 64, 128, 255))
MID_N = 4096
MID_ROOF = (255, 4096)  # the point whose kernel the mid leg's roofline names


def bench_mid(torch, r9k, inputs, dev, reps, points=MID_POINTS):
    res = []
    for K, N in ((4096, MID_N), (14336, MID_N)):
        Ms = [M for M, k in points if k == K]
        if not Ms:
            continue
        a = dev(inputs.activations(2, 255, K, outliers=True))
        copies = weight_copies(torch, r9k, dev, inputs.weights(2, N, K))
        copies = [(r9k.pack_weight(wq), ws) for wq, ws in copies]  # fragment order, packed at load
        C = len(copies)
        for M in Ms:
            wsp = torch.zeros(r9k.gemm_fp8_block_workspace(M, K, N), dtype=torch.uint8, device="cuda")
            am = a[:M].contiguous()
            c_out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            calls = [lambda c=c: r9k.gemm_fp8_block_qa_packed(am, copies[c][0], copies[c][1], c=c_out,
                                                              workspace=wsp)
                     for c in range(C)]
            for f in calls:
                f()
            g = capture(torch, calls)
            tm = Timer(torch)
            warm_graph(tm, g)
            ms, tr = median_of_trials(lambda: tm.run(lambda i: g.replay(), reps) / C)
            gbs = gemm_bytes(M, K, N) / (ms * 1e-3) / 1e9
            tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            log(f"mid M={M} K={K} N={N}: {ms * 1e3:.2f} us, {gbs:.0f} GB/s, {tf:.0f} TFLOP/s")
            res.append(dict(M=M, K=K, N=N, us=ms * 1e3, GBs=gbs, hbm_frac=gbs / HBM_PEAK_GBS, TFLOPs=tf,
                            kernel=KERNEL_NAMES.get(r9k.gemm_fp8_block_plan(M, K, N, True)[0]),
                            trials_us=[t * 1e3 for t in tr]))
        del copies
        torch.cuda.empty_cache()
    return res


def bench_moe(torch, r9k, inputs, dev, reps):
    T, H, E, I, k = 16, 2048, 128, 768, 8
    x, logits, w13, w2 = inputs.moe_inputs(0, T, H, E, I)
    host = dict(x=x, logits=logits, k=k, H=H, I=I, E=E, w13=w13, w2=w2)
    logits_d = torch.from_numpy(logits).cuda()
    ids_d, tw_d = r9k.moe_route(logits_d, k)  # the library's one-launch routing
    ids = ids_d.cpu().numpy()
    q13, s13 = r9k.quant_weight(dev(w13.reshape(E * 2 * I, H)))
    q2, s2 = r9k.quant_weight(dev(w2.reshape(E * H, I)))
    # fragment-order expert weights (packed once at load, not timed)
    q13 = r9k.pack_weight(q13)
    q2 = r9k.pack_weight(q2)
    sets = [(q13, s13, q2, s2), (q13.clone(), s13.clone(), q2.clone(), s2.clone())]
    x_d = dev(x)
    shared_d = dev(inputs.activations(1, T, H, outliers=False))  # a stand-in for the shared expert's output
    wsp = torch.zeros(r9k.moe_fp8_decode_workspace(T, H, E, I, k), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    touched = len(np.unique(ids))
    per_expert = 2 * I * H + 4 * (2 * I // 128) * (H // 128) + H * I + 4 * (H // 128) * (I // 128)
    nbytes = touched * per_expert + 2 * T * H * 2 + T * k * 8
    res = {}
    # routing alone: a graph of back-to-back launches
    rcalls = [lambda: r9k.moe_route(logits_d, k, ids=ids_d, w=tw_d)] * 20
    g = capture(torch, rcalls)
    tm = Timer(torch)
    warm_graph(tm, g)
    ms, tr = median_of_trials(lambda: tm.run(lambda i: g.replay(), reps) / len(rcalls))
    res["route"] = dict(us=ms * 1e3, T=T, E=E, topk=k, trials_us=[t * 1e3 for t in tr])
    log(f"moe route T={T} E={E} top-{k}: {res['route']['us']:.2f} us")
    for fused in (True, False):
        calls = [lambda s=s: r9k.moe_fp8_decode(x_d, ids_d, tw_d, s[0].view(E, 2 * I, H),
                                                s[1].view(E, 2 * I // 128, H // 128), s[2].view(E, H, I),
                                                s[3].view(E, H // 128, I // 128), out=out, workspace=wsp,
                                                fused=fused, packed=True) for s in sets]
        for f in calls:
            f()
        g = capture(torch, calls)
        tm = Timer(torch)
        warm_graph(tm, g)
        ms, tr = median_of_trials(lambda: tm.run(lambda i: g.replay(), reps) / len(sets))
        gbs = nbytes / (ms * 1e-3) / 1e9
        log(f"moe fused={fused}: {ms * 1e3:.1f} us, {gbs:.0f} GB/s over {touched} touched experts")
        res["fused" if fused else "three_launch"] = dict(us=ms * 1e3, GBs=gbs, hbm_frac=gbs / HBM_PEAK_GBS,
                                                         trials_us=[t * 1e3 for t in tr])
    # the fused path with the shared expert's term folded into the combine
    calls = [lambda s=s: r9k.moe_fp8_decode(x_d, ids_d, tw_d, s[0].view(E, 2 * I, H),
                                            s[1].view(E, 2 * I // 128, H // 128), s[2].view(E, H, I),
                                            s[3].view(E, H // 128, I // 128), out=out, workspace=wsp,
                                            fused=True, packed=True, shared=shared_d) for s in sets]
    for f in calls:
        f()
    g = capture(torch, calls)
    tm = Timer(torch)
    warm_graph(tm, g)
    ms, tr = median_of_trials(lambda: tm.run(lambda i: g.replay(), reps) / len(sets))
    res["fused_shared"] = dict(us=ms * 1e3, GBs=nbytes / (ms * 1e-3) / 1e9, trials_us=[t * 1e3 for t in tr])
    log(f"moe fused with the shared expert's term: {ms * 1e3:.1f} us")
    res.update(workload=f"T={T}, H={H}, E={E}, I={I}, top-{k}", touched_experts=touched, bytes=nbytes)
    host["nbytes"] = nbytes
    return res, host


def bench_single_token(torch, r9k, inputs, dev, reps):
    """The single decode token: A 1x512 (N(0,1), no outliers), W 1024x512, seed 0,
    row-major weights, fused act quant.  Everything sits in cache; this is the
    call's latency, in a graph of back-to-back calls and as eager calls."""
    M, K, N = 1, 512, 1024
    a = dev(inputs.activations(0, M, K, outliers=False))
    wq, ws = r9k.quant_weight(dev(inputs.weights(0, N, K)))
    wsp = torch.zeros(max(r9k.gemm_fp8_block_workspace(M, K, N), 256), dtype=torch.uint8, device="cuda")
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    one = lambda: r9k.gemm_fp8_block_qa(a, wq, ws, c=c, workspace=wsp)
    one()
    calls = [one] * 50
    g = capture(torch, calls)
    tm = Timer(torch)
    warm_graph(tm, g)
    ms, tr = median_of_trials(lambda: tm.run(lambda i: g.replay(), reps) / len(calls))
    ems, etr = median_of_trials(lambda: tm.run(lambda i: one(), 200))
    log(f"single token {M}x{K}x{N}: {ms * 1e3:.2f} us a call in a graph, {ems * 1e3:.2f} us eager")
    return dict(workload=f"M={M}, K={K}, N={N}, seed 0, fused act quant, row-major weights", us=ms * 1e3,
                eager_us=ems * 1e3, trials_us=[t * 1e3 for t in tr], eager_trials_us=[t * 1e3 for t in etr],
                kernel=KERNEL_NAMES.get(r9k.gemm_fp8_block_plan(M, K, N)[0]))


# ---- the oracle beside each leg (CPU, the host's cores) ----

def cpu_prefill(ora, inputs, rows=512):
    M, K, N = 4096, 4096, 12288
    a = inputs.activations(1, M, K, outliers=True)[:rows]
    wq, ws = ora.quant_weight(inputs.weights(1, N, K))
    t, n = cpu_seconds(lambda: ora.gemm_block_qa(a, wq, ws))
    return dict(value=2.0 * rows * K * N / t / 1e12, unit="TFLOP/s", cores=ora.threads(), kind="oracle",
                seconds=t, repeats=n,
                sample=f"the first {rows} of the {M} rows (K={K}, N={N}): oracle act quant + exact block GEMM, "
                       f"weight quant not timed; TFLOP/s of the sample")


def cpu_mid(ora, inputs):
    M, K, N = 255, 4096, 4096
    a = inputs.activations(2, 255, K, outliers=True)
    wq, ws = ora.quant_weight(inputs.weights(2, N, K))
    t, n = cpu_seconds(lambda: ora.gemm_block_qa(a, wq, ws))
    return dict(value=gemm_bytes(M, K, N) / t / 1e9, unit="GB/s", tflops=2.0 * M * K * N / t / 1e12,
                cores=ora.threads(), kind="oracle", seconds=t, repeats=n,
                sample=f"the M={M}, K={K}, N={N} point in full: oracle act quant + exact block GEMM, weight "
                       f"quant not timed; GB/s of the same algorithmic bytes as the GPU figure")


def moe_oracle_args(ora, host):
    """The oracle's MoE decode arguments for the workload: routed by the oracle, with
    only the experts the routing touches quantised (by the oracle) and the ids
    renumbered into that compact set; the other experts are never read."""
    x, logits, k = host["x"], host["logits"], host["k"]
    H = x.shape[1]
    E, I = host["E"], host["I"]
    ids, w = ora.moe_route(logits, k)
    touched = np.unique(ids)
    remap = np.full(E, -1, np.int64)
    remap[touched] = np.arange(len(touched))
    w13, w2 = host["w13"][touched], host["w2"][touched]
    q13, s13 = ora.quant_weight(w13.reshape(-1, H))
    q2, s2 = ora.quant_weight(w2.reshape(-1, I))
    Et = len(touched)
    return (x, remap[ids].astype(ids.dtype), w, q13.reshape(Et, 2 * I, H), s13.reshape(Et, 2 * I // 128, H // 128),
            q2.reshape(Et, H, I), s2.reshape(Et, H // 128, I // 128))


def cpu_moe(ora, host):
    x, k = host["x"], host["k"]
    T = x.shape[0]
    args = moe_oracle_args(ora, host)  # setup, not timed
    Et = args[3].shape[0]
    t, n = cpu_seconds(lambda: ora.moe_decode(*args))
    return dict(value=host["nbytes"] / t / 1e9, unit="GB/s", cores=ora.threads(), kind="oracle", seconds=t,
                repeats=n, sample=f"the workload in full (T={T}, top-{k}, the {Et} touched experts): oracle "
                                  f"gate_up + silu*up + row quant + down + weighted sum, routing and weight quant "
                                  f"not timed; GB/s over the same bytes as the GPU figure")


def cpu_single_token(ora, inputs):
    M, K, N = 1, 512, 1024
    a = inputs.activations(0, M, K, outliers=False)
    wq, ws = ora.quant_weight(inputs.weights(0, N, K))
    t, n = cpu_seconds(lambda: ora.gemm_block_qa(a, wq, ws), max_runs=20)
    return dict(value=t * 1e6, unit="us", cores=ora.threads(), kind="oracle", repeats=n,
                sample=f"the M={M}, K={K}, N={N} call in full (weight quant not timed)")


BENCH_LIB = os.path.join(ROOT, "block_scaled_fp8_r9k_amd", "libr9k_bench.so")


def hbm_read_ceiling(torch, reps, nbytes=DECODE_K * DECODE_N):
    """The bandwidth ceiling beside the decode roofline: a plain read (no compute) of
    the decode weight's byte count, rotated over the same number of copies and timed
    the same way (graphs of back-to-back launches), in two access patterns
    (libr9k_bench.so: a grid-stride read, and 16 KiB slabs per wave with staggered
    starts); median of 3 trials each."""
    import ctypes
    lib = ctypes.CDLL(BENCH_LIB)
    lib.r9kb_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    n = max(2, min(16, -(-ROTATE_BYTES // nbytes)))
    bufs = [torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda") for _ in range(n)]
    out = torch.zeros(512, dtype=torch.int32, device="cuda")
    res = {}
    for mode, name in ((0, "grid_stride"), (1, "slabs_16k_staggered")):
        def one(i, mode=mode):
            rc = lib.r9kb_hbm_read(bufs[i % n].data_ptr(), nbytes, mode, out.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"r9kb_hbm_read mode {mode}: {rc}")
        calls = [lambda i=i: one(i) for i in range(2 * n)]
        for f in calls:
            f()
        g = capture(torch, calls)
        tm = Timer(torch)
        warm_graph(tm, g)
        ms, tr = median_of_trials(lambda: tm.run(lambda i: g.replay(), reps) / len(calls))
        res[name] = dict(us=ms * 1e3, GBs=nbytes / (ms * 1e-3) / 1e9, trials_us=[t * 1e3 for t in tr])
        log(f"plain read of {nbytes / 1e6:.1f} MB ({name}): {ms * 1e3:.2f} us, {res[name]['GBs']:.0f} GB/s")
    best = max(v["GBs"] for v in res.values())
    del bufs
    torch.cuda.empty_cache()
    return dict(bytes=nbytes, copies=n, best_GBs=best, frac_of_peak=best / HBM_PEAK_GBS, **res)


def copy_bandwidth(torch):
    """Context only: a plain device copy of 1 GiB (read + write bytes / time)."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    tm = Timer(torch)
    tm.run(lambda i: dst.copy_(src), 2)
    ms = tm.run(lambda i: dst.copy_(src), 10)
    del src, dst
    return 2 * n / (ms * 1e-3) / 1e9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", default="decode,prefill,mid,moe,single_token,bf16a")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mid-points", default=None,
                    help="mid leg points as MxK,... (N=4096; default: M in 32,64,128,255 at K=4096 and 14336)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one MI355X: the path is single-GPU (no collectives); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    which = set(args.only.split(","))

    import torch
    import block_scaled_fp8_r9k_amd as r9k
    import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    r9k.lib()

    def dev(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    line = dict(metric="block-fp8 GEMM: HBM GB/s (% peak) at M<=16; fp8 TFLOPS (% MFMA peak) at M=4096",
                value=None, unit="GB/s", n_gpus=1, steps=args.steps, warmup=args.warmup, ms_per_step=None,
                higher_is_better=True, scaling="weak", vs_baseline=None, dtype="fp8_e4m3", data="synthetic",
                config=dict(workload="decode-width sweep: M in {1,2,4,8,16}, K=4096, N=14336, bf16 act quantised "
                                     "per token in groups of 128 inside the GEMM, fp8 e4m3 weights with 128x128 "
                                     "fp32 block scales, bf16 out", M=list(DECODE_M), K=DECODE_K, N=DECODE_N))
    if "decode" in which:
        drm = bench_decode(torch, r9k, inputs, dev, args.steps, args.warmup, packed=False)
        line["per_m_row_major"] = {str(M): v for M, v in drm["per_m"].items()}
        line["value_row_major"] = drm["step_bytes"] / (drm["ms_step"] * 1e-3) / 1e9
        d = bench_decode(torch, r9k, inputs, dev, args.steps, args.warmup, packed=True)
        line["value"] = d["step_bytes"] / (d["ms_step"] * 1e-3) / 1e9
        line["ms_per_step"] = d["ms_step"]
        line["hbm_frac"] = line["value"] / HBM_PEAK_GBS
        line["roofline"] = dict(bound="hbm", achieved=d["achieved"], peak=HBM_PEAK_GBS, unit="GB/s",
                                frac=d["achieved"] / HBM_PEAK_GBS, traffic=traffic_from_profiles(),
                                kernel="k_gemm_decode (activation quant in the A-load, fragment-order "
                                       "weights), average over the sweep's five launches",
                                bytes_per_launch=d["bytes_avg"], us_per_launch=d["us_avg"])
        line["per_m"] = {str(M): v for M, v in d["per_m"].items()}
        if os.path.exists(BENCH_LIB):
            ceil = hbm_read_ceiling(torch, max(5, args.steps // 20))
            line["hbm_read_ceiling"] = ceil
            line["roofline"]["frac_of_read_ceiling"] = d["achieved"] / ceil["best_GBs"]
        if not args.no_cpu_baseline:
            import oracle
            log("cpu baseline (oracle) ...")
            line["cpu_baseline"] = cpu_baseline(oracle, d["a_bits"], d["w_bits"], d["step_bytes"])
    reps = max(5, args.steps // 20)
    moe_host = None
    if "prefill" in which:
        line["prefill"] = bench_prefill(torch, r9k, inputs, dev, reps)
    if "mid" in which:
        points = MID_POINTS
        if args.mid_points:
            points = tuple(tuple(int(v) for v in p.split("x")) for p in args.mid_points.split(","))
        line["mid"] = dict(points=bench_mid(torch, r9k, inputs, dev, reps, points))
        roof = [p for p in line["mid"]["points"] if (p["M"], p["K"]) == MID_ROOF]
        if roof:
            p = roof[0]
            line["mid"]["roofline"] = dict(
                bound="hbm", achieved=p["GBs"], peak=HBM_PEAK_GBS, unit="GB/s", frac=p["GBs"] / HBM_PEAK_GBS,
                traffic=traffic_from_profiles(MID_COUNTERS, ("gemm_mid.hip", "quant.hip")),
                kernel=f"k_quant_act + k_gemm_mid per fused call at M={p['M']}, K={p['K']}, N={p['N']}",
                bytes_per_launch=gemm_bytes(p["M"], p["K"], p["N"]), us_per_launch=p["us"])
    if "moe" in which:
        line["moe"], moe_host = bench_moe(torch, r9k, inputs, dev, reps)
    if "single_token" in which:
        line["single_token"] = bench_single_token(torch, r9k, inputs, dev, reps)
    if "bf16a" in which:
        line["bf16a"] = bench_bf16a(torch, r9k, inputs, dev, reps)
    if not args.no_cpu_baseline:
        import oracle
        log("cpu baselines of the other legs (oracle) ...")
        if "prefill" in which:
            line["prefill"]["cpu_baseline"] = cpu_prefill(oracle, inputs)
        if "mid" in which:
            line["mid"]["cpu_baseline"] = cpu_mid(oracle, inputs)
        if "moe" in which:
            line["moe"]["cpu_baseline"] = cpu_moe(oracle, moe_host)
        if "single_token" in which:
            line["single_token"]["cpu_baseline"] = cpu_single_token(oracle, inputs)
    moe_host = None
    line["copy_GBs_context"] = copy_bandwidth(torch)
    line["kernel_source_hash"] = kernel_source_hash()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
