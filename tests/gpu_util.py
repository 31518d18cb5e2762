"""Helpers for the GPU parity tests: numpy <-> device tensors and comparisons.

The GPU side runs through the C ABI (the block_scaled_fp8_r9k_amd binding);
the expected values come from the oracle on the same seeded inputs.
"""
import sys

import numpy as np
import torch


def say(*a):
    """Name the case before each GPU step, flushed, so a failure names it."""
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, dtype=None) -> torch.Tensor:
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(x)
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def assert_bits_equal(a: np.ndarray, b: np.ndarray, what: str):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if a.dtype == np.float32:
        a = a.view(np.uint32)
        b = np.asarray(b, np.float32).view(np.uint32)
    bad = np.argwhere(a != b)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {tuple(bad[0])}: {a[tuple(bad[0])]} vs {b[tuple(bad[0])]}"


def assert_close(ora, gpu_bits: np.ndarray, oracle_f64: np.ndarray, what: str, rms_over=None):
    ok, ratio, bound = ora.within_tolerance(gpu_bits, oracle_f64, rms_over=rms_over)
    if not ok:
        g = ora.bf16_value(gpu_bits).astype(np.float64)
        err = np.abs(g - oracle_f64)
        idx = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(f"{what}: worst |gpu-oracle|/bound = {ratio:.3g} at {idx}: gpu {g[idx]!r} "
                             f"oracle {oracle_f64[idx]!r} bound {bound[idx]!r}")
    return ratio
