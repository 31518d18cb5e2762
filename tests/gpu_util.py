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


def assert_layouts_agree(ora, a_bits: np.ndarray, b_bits: np.ndarray, what: str):
    """Two bf16 results of the same GEMM on the two weight layouts.  The decode planner may slice K
    differently for fragment-order and row-major weights (each layout's fastest launch), and a different
    slicing sums the fp32 partials in a different order.  Two fp32 sums of the same terms in different
    orders differ by a few fp32 roundings of the terms' size, which is far below a bf16 ulp of a typical
    output but not of one that nearly cancels; so the results agree to within one bf16 ulp plus 2^-16 of
    the output's RMS (about 2^7 fp32 roundings of a typical term), and only on a small share of the
    outputs do they differ at all.  Where the plans coincide they are equal."""
    a = ora.bf16_value(a_bits).astype(np.float64)
    b = ora.bf16_value(b_bits).astype(np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    diff = np.abs(a - b)
    bound = ora.bf16_ulp(b) + 2.0 ** -16 * np.sqrt(np.mean(b * b))
    bad = np.argwhere(diff > bound)
    assert bad.size == 0, f"{what}: {len(bad)} outputs differ by more than one bf16 ulp, first at {tuple(bad[0])}"
    n_diff = int(np.count_nonzero(a_bits != b_bits))
    assert n_diff <= max(2, a.size // 1000), f"{what}: {n_diff} of {a.size} outputs differ"
