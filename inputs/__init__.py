"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

A module of its own, outside the GPU library's package and the oracle, so that
neither side imports the other to get its inputs.

This module holds none of the method's arithmetic: it draws random numbers,
rounds them to bf16 with torch's own conversion and picks outlier channels.
Quantisation, GEMMs, MoE routing and everything else the method computes
happen in the GPU library or in the oracle, each on its own.

Recipe (the workloads of the release pages' decode/prefill GEMMs):
  * activations: z ~ N(0, 1) in fp32; a fixed set of round(0.01 * K) channels
    (the same for every row) is multiplied by 20 before rounding to bf16;
  * weights: fp32(0.02 * z), rounded to bf16; quantised per 128x128 block by
    whichever side consumes them;
  * MoE: router logits ~ N(0, 1) in fp32 (the routing itself, top-k with
    renormalised softmax weights, is a step of the method).
Streams: numpy PCG64 seeded from SeedSequence([seed, tag]), one tag per tensor.
"""
from __future__ import annotations

import numpy as np
import torch

TAG_A, TAG_W, TAG_OUTLIER, TAG_LOGITS, TAG_X, TAG_W13, TAG_W2 = 1, 2, 3, 4, 5, 6, 7


def rng(seed: int, tag: int, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, sub])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (torch's round-to-nearest-even conversion); bits as uint16."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def outlier_channels(seed: int, K: int, frac: float = 0.01) -> np.ndarray:
    n = int(round(frac * K))
    return np.sort(rng(seed, TAG_OUTLIER).permutation(K)[:n])


def activations(seed: int, M: int, K: int, outliers: bool = True, tag: int = TAG_A) -> np.ndarray:
    """bf16 bits [M, K]: N(0,1), with 1% of the channels x20 when outliers is set."""
    z = rng(seed, tag).standard_normal((M, K), dtype=np.float32)
    if outliers:
        z[:, outlier_channels(seed, K)] *= np.float32(20.0)
    return to_bf16_bits(z)


def weights(seed: int, N: int, K: int, tag: int = TAG_W, sub: int = 0) -> np.ndarray:
    """bf16 bits [N, K] of fp32(0.02 * z), z ~ N(0,1)."""
    z = rng(seed, tag, sub).standard_normal((N, K), dtype=np.float32)
    return to_bf16_bits(z * np.float32(0.02))


def moe_inputs(seed: int, T: int, H: int, E: int, I: int):
    """x [T,H] bf16, router logits [T,E] f32, w13 [E,2I,H] bf16, w2 [E,H,I] bf16."""
    x = activations(seed, T, H, outliers=True, tag=TAG_X)
    logits = router_logits(seed, T, E)
    w13 = np.empty((E, 2 * I, H), np.uint16)
    w2 = np.empty((E, H, I), np.uint16)
    for e in range(E):
        w13[e] = weights(seed, 2 * I, H, tag=TAG_W13, sub=e)
        w2[e] = weights(seed, H, I, tag=TAG_W2, sub=e)
    return x, logits, w13, w2


def router_logits(seed: int, T: int, E: int) -> np.ndarray:
    """Router logits [T, E] fp32, N(0, 1)."""
    return rng(seed, TAG_LOGITS).standard_normal((T, E), dtype=np.float32)


def quant_edge_groups() -> np.ndarray:
    """Adversarial activation rows (bf16 bits, K = 128 * 12): constant groups,
    all-zero and negative-zero groups, subnormal-only groups, a single outlier,
    powers of two, values straddling e4m3 rounding midpoints, and groups whose
    maximum sits at the last or first position."""
    rows = []
    f = lambda v: np.asarray(v, np.float32)
    g = np.zeros(128, np.float32); rows.append(g)                          # all +0
    g = -np.zeros(128, np.float32); rows.append(g)                         # all -0
    g = np.full(128, 3.0, np.float32); rows.append(g)                      # constant
    g = np.full(128, -1e-41, np.float32); g[5] = 1e-41; rows.append(g)     # subnormal bf16 only
    g = np.zeros(128, np.float32); g[77] = -5.0; rows.append(g)            # single value
    g = f(2.0 ** np.arange(-64, 64)); rows.append(g)                       # powers of two
    g = np.linspace(-1.0, 1.0, 128, dtype=np.float32); rows.append(g)
    g = np.linspace(0.0, 448.0, 128, dtype=np.float32); rows.append(g)     # already on a 448 scale
    mids = np.array([(1 + (2 * m + 1) / 16) * 2.0 ** e for e in range(-9, 9) for m in range(8)], np.float64)
    mids = mids[mids < 448.0][-127:]
    g = f(np.concatenate([mids[:127], [448.0]])); rows.append(g)           # e4m3 midpoints at unit scale
    g = f(np.concatenate([mids[:127] * 3.0, [448.0 * 3.0]])); rows.append(g)
    g = np.ones(128, np.float32); g[-1] = 1e30; rows.append(g)             # max last
    g = np.ones(128, np.float32); g[0] = -1e-30; g[1:] = 1e-33; rows.append(g)  # max first, tiny
    row = np.concatenate(rows)[None, :]
    return to_bf16_bits(row)
