"""CPU oracle for the block-scaled fp8 GEMM path (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package.  The GPU library (``block_scaled_fp8_r9k_amd``) never imports it, and
it imports nothing from there.  The arithmetic lives in ``r9k_oracle.c``
(plain C, binary64 wherever the method does not fix an fp32 step); this module
only marshals numpy arrays into it.

What each function computes, and the page passage it follows, is stated in the
C source next to the function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from ctypes import POINTER, c_double, c_float, c_int, c_int64, c_uint8, c_uint16, c_int32

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "r9k_oracle.c")
_LIB = os.path.join(_HERE, "libr9k_oracle.so")
_CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-pthread"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE binary32/binary64 on x86-64 SSE)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def threads() -> int:
    """Host threads the oracle uses (all cores the process may run on)."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_LIB)
        u8p, u16p, f32p, f64p, i32p, i64p = (POINTER(c_uint8), POINTER(c_uint16), POINTER(c_float),
                                            POINTER(c_double), POINTER(c_int32), POINTER(c_int64))
        L.ora_e4m3_value.argtypes = [c_uint8]
        L.ora_e4m3_value.restype = c_double
        L.ora_e4m3_encode.argtypes = [c_float]
        L.ora_e4m3_encode.restype = c_uint8
        L.ora_e4m3_encode_array.argtypes = [f32p, c_int64, u8p, c_int]
        L.ora_bf16_value.argtypes = [c_uint16]
        L.ora_bf16_value.restype = c_float
        L.ora_bf16_round.argtypes = [c_double]
        L.ora_bf16_round.restype = c_uint16
        L.ora_bf16_round_array.argtypes = [f64p, c_int64, u16p, c_int]
        L.ora_quant_act.argtypes = [u16p, c_int64, c_int64, u8p, f32p, c_int]
        L.ora_quant_weight.argtypes = [u16p, c_int64, c_int64, u8p, f32p, c_int]
        L.ora_gemm_block.argtypes = [u8p, f32p, c_int64, c_int64, u8p, f32p, c_int64, u16p, f64p, c_int]
        L.ora_gemm_block_at.argtypes = [u8p, f32p, c_int64, c_int64, u8p, f32p, c_int64, i64p, i64p, c_int64,
                                        u16p, f64p, c_int]
        L.ora_moe_decode.argtypes = [u16p, c_int64, c_int64, i32p, f32p, c_int64, u8p, f32p, u8p, f32p, c_int64,
                                     c_int64, u16p, u16p, u16p, u8p, f32p, f64p, c_int]
        L.ora_moe_silu_mul.argtypes = [u16p, c_int64, c_int64, u16p]
        L.ora_moe_down_from_h.argtypes = [u16p, c_int64, c_int64, i32p, f32p, c_int64, u8p, f32p, c_int64, c_int64,
                                          u16p, u8p, f32p, f64p, c_int]
        L.ora_moe_route.argtypes = [f32p, c_int64, c_int64, c_int64, i32p, f32p]
        L.ora_gemm_block_bf16a.argtypes = [u16p, c_int64, c_int64, u8p, f32p, c_int64, u16p, f64p, c_int]
        L.ora_moe_fold.argtypes = [f64p, i32p, f32p, c_int64, c_int64, c_int64, c_int64, u16p, f32p, u16p]
        _lib = L
    return _lib


def _p(a: np.ndarray | None, ctype):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(POINTER(ctype))


def _u16(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return np.ascontiguousarray(a, dtype=np.uint16)


# ---------------------------------------------------------------- codecs ----

def e4m3_value(code: int) -> float:
    return lib().ora_e4m3_value(int(code))


def e4m3_table() -> np.ndarray:
    """Values of all 256 codes (NaN at 0x7F and 0xFF)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, dtype=np.uint8)
    lib().ora_e4m3_encode_array(_p(x, c_float), x.size, _p(out, c_uint8), threads())
    return out


def bf16_value(b) -> np.ndarray:
    b = _u16(b)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    lib().ora_bf16_round_array(_p(x, c_double), x.size, _p(out, c_uint16), threads())
    return out


# ----------------------------------------------------------------- quant ----

def quant_act(a_bf16) -> tuple[np.ndarray, np.ndarray]:
    """Per-row group-128 activation quant: a [M,K] bf16 bits -> (codes [M,K], scales [M,K/128])."""
    a = _u16(a_bf16)
    M, K = a.shape
    assert K % 128 == 0
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, K // 128), np.float32)
    lib().ora_quant_act(_p(a, c_uint16), M, K, _p(q, c_uint8), _p(s, c_float), threads())
    return q, s


def quant_weight(w_bf16) -> tuple[np.ndarray, np.ndarray]:
    """128x128 block weight quant: w [N,K] bf16 bits -> (codes [N,K], scales [N/128,K/128])."""
    w = _u16(w_bf16)
    N, K = w.shape
    assert N % 128 == 0 and K % 128 == 0
    q = np.empty((N, K), np.uint8)
    s = np.empty((N // 128, K // 128), np.float32)
    lib().ora_quant_weight(_p(w, c_uint16), N, K, _p(q, c_uint8), _p(s, c_float), threads())
    return q, s


# ------------------------------------------------------------------ gemm ----

def gemm_block(aq, as_, wq, ws, want_f64: bool = False):
    """C = bf16(sum_g P_g * as * ws) from codes and scales.  Returns bf16 bits [M,N]
    (and the unrounded binary64 values if want_f64)."""
    aq = np.ascontiguousarray(aq, np.uint8)
    as_ = np.ascontiguousarray(as_, np.float32)
    wq = np.ascontiguousarray(wq, np.uint8)
    ws = np.ascontiguousarray(ws, np.float32)
    M, K = aq.shape
    N = wq.shape[0]
    c = np.empty((M, N), np.uint16)
    c64 = np.empty((M, N), np.float64) if want_f64 else None
    lib().ora_gemm_block(_p(aq, c_uint8), _p(as_, c_float), M, K, _p(wq, c_uint8), _p(ws, c_float), N,
                         _p(c, c_uint16), _p(c64, c_double), threads())
    return (c, c64) if want_f64 else c


def gemm_block_at(aq, as_, wq, ws, ms, ns, want_f64: bool = False):
    """The same definition at sampled positions (ms[i], ns[i])."""
    aq = np.ascontiguousarray(aq, np.uint8)
    as_ = np.ascontiguousarray(as_, np.float32)
    wq = np.ascontiguousarray(wq, np.uint8)
    ws = np.ascontiguousarray(ws, np.float32)
    ms = np.ascontiguousarray(ms, np.int64)
    ns = np.ascontiguousarray(ns, np.int64)
    M, K = aq.shape
    N = wq.shape[0]
    c = np.empty(ms.shape, np.uint16)
    c64 = np.empty(ms.shape, np.float64) if want_f64 else None
    lib().ora_gemm_block_at(_p(aq, c_uint8), _p(as_, c_float), M, K, _p(wq, c_uint8), _p(ws, c_float), N,
                            _p(ms, c_int64), _p(ns, c_int64), ms.size, _p(c, c_uint16), _p(c64, c_double),
                            threads())
    return (c, c64) if want_f64 else c


def gemm_block_qa(a_bf16, wq, ws, want_f64: bool = False):
    """The fused form: activation quant then the block GEMM (one definition for every M)."""
    aq, as_ = quant_act(a_bf16)
    return gemm_block(aq, as_, wq, ws, want_f64)


def gemm_block_bf16a(a_bf16, wq, ws, want_f64: bool = False):
    """The bf16-activation variant: C = bf16(sum_g ws * sum_k a * dec(w)), no activation quant; see
    ora_gemm_block_bf16a."""
    a = _u16(a_bf16)
    wq = np.ascontiguousarray(wq, np.uint8)
    ws = np.ascontiguousarray(ws, np.float32)
    M, K = a.shape
    N = wq.shape[0]
    c = np.empty((M, N), np.uint16)
    c64 = np.empty((M, N), np.float64) if want_f64 else None
    lib().ora_gemm_block_bf16a(_p(a, c_uint16), M, K, _p(wq, c_uint8), _p(ws, c_float), N, _p(c, c_uint16),
                               _p(c64, c_double), threads())
    return (c, c64) if want_f64 else c


# ------------------------------------------------------------------- moe ----

def moe_decode(x, ids, w, w13q, w13s, w2q, w2s, intermediates: bool = False):
    """MoE decode for T tokens: see ora_moe_decode in the C source for the definition."""
    x = _u16(x)
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.ascontiguousarray(w, np.float32)
    w13q = np.ascontiguousarray(w13q, np.uint8)
    w13s = np.ascontiguousarray(w13s, np.float32)
    w2q = np.ascontiguousarray(w2q, np.uint8)
    w2s = np.ascontiguousarray(w2s, np.float32)
    T, H = x.shape
    topk = ids.shape[1]
    E, twoI, _ = w13q.shape
    I = twoI // 2
    P = T * topk
    out = np.empty((T, H), np.uint16)
    inter = None
    if intermediates:
        inter = dict(gu=np.empty((P, 2 * I), np.uint16), h=np.empty((P, I), np.uint16),
                     hq=np.empty((P, I), np.uint8), hs=np.empty((P, I // 128), np.float32),
                     y=np.empty((P, H), np.float64))
    g = (lambda k, t: _p(inter[k], t)) if inter else (lambda k, t: None)
    lib().ora_moe_decode(_p(x, c_uint16), T, H, _p(ids, c_int32), _p(w, c_float), topk, _p(w13q, c_uint8),
                         _p(w13s, c_float), _p(w2q, c_uint8), _p(w2s, c_float), E, I, _p(out, c_uint16),
                         g("gu", c_uint16), g("h", c_uint16), g("hq", c_uint8), g("hs", c_float), g("y", c_double),
                         threads())
    return (out, inter) if intermediates else out


def moe_silu_mul(gu):
    """h = bf16(silu(gate) * up) per pair from gu [P, 2I] (bf16 bits) -> h [P, I]."""
    gu = _u16(gu)
    P, twoI = gu.shape
    h = np.empty((P, twoI // 2), np.uint16)
    lib().ora_moe_silu_mul(_p(gu, c_uint16), P, twoI // 2, _p(h, c_uint16))
    return h


def moe_down_from_h(h, ids, w, w2q, w2s, intermediates: bool = False):
    """Down stage + weighted combine from given h rows [T*topk, I] (bf16 bits)."""
    h = _u16(h)
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.ascontiguousarray(w, np.float32)
    w2q = np.ascontiguousarray(w2q, np.uint8)
    w2s = np.ascontiguousarray(w2s, np.float32)
    T, topk = ids.shape
    E, H, I = w2q.shape
    P = T * topk
    out = np.empty((T, H), np.uint16)
    hq = np.empty((P, I), np.uint8)
    hs = np.empty((P, I // 128), np.float32)
    y = np.empty((P, H), np.float64)
    lib().ora_moe_down_from_h(_p(h, c_uint16), T, H, _p(ids, c_int32), _p(w, c_float), topk, _p(w2q, c_uint8),
                              _p(w2s, c_float), E, I, _p(out, c_uint16), _p(hq, c_uint8), _p(hs, c_float),
                              _p(y, c_double), threads())
    return (out, dict(hq=hq, hs=hs, y=y)) if intermediates else out


def moe_route(logits, topk: int):
    """Routing: logits [T, E] fp32 -> (ids [T, topk] int32, weights [T, topk] fp32); see ora_moe_route."""
    logits = np.ascontiguousarray(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, topk), np.int32)
    w = np.empty((T, topk), np.float32)
    lib().ora_moe_route(_p(logits, c_float), T, E, topk, _p(ids, c_int32), _p(w, c_float))
    return ids, w


def moe_fold(y, ids, w, E: int, shared=None, shared_w=None):
    """out [T, H] bf16 bits = the routed sum of y [T*topk, H] plus the shared term; see ora_moe_fold."""
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.ascontiguousarray(w, np.float32)
    T, topk = ids.shape
    y = np.ascontiguousarray(y, np.float64).reshape(T * topk, -1)
    H = y.shape[1]
    s = None if shared is None else _u16(shared)
    g = None if shared_w is None else np.ascontiguousarray(shared_w, np.float32)
    out = np.empty((T, H), np.uint16)
    lib().ora_moe_fold(_p(y, c_double), _p(ids, c_int32), _p(w, c_float), T, topk, H, E,
                       _p(s, c_uint16), _p(g, c_float), _p(out, c_uint16))
    return out


# ------------------------------------------------------------ comparison ----

def bf16_ulp(x64: np.ndarray) -> np.ndarray:
    """One bf16 ulp at each value: 2^(floor(log2|x|) - 7) for normal |x|, the
    smallest bf16 subnormal (2^-133) at 0 and below 2^-126."""
    ax = np.abs(np.asarray(x64, np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, -126.0)
    ulp = np.ldexp(1.0, (e - 7).astype(np.int64))
    return np.where(ax > 0, ulp, 2.0 ** -133)


def within_tolerance(gpu_bf16, oracle_f64, rms_over=None):
    """Elementwise |gpu - oracle| <= 1e-2 * RMS(oracle) + 1 bf16 ulp(oracle).

    The RMS is taken over ``rms_over`` (the whole output of the call) when
    given, else over ``oracle_f64``.  Returns (ok, worst ratio, bound array)."""
    g = bf16_value(gpu_bf16).astype(np.float64)
    o = np.asarray(oracle_f64, np.float64)
    base = o if rms_over is None else np.asarray(rms_over, np.float64)
    rms = float(np.sqrt(np.mean(base * base))) if base.size else 0.0
    bound = 1e-2 * rms + bf16_ulp(o)
    err = np.abs(g - o)
    ratio = float(np.max(err / bound)) if err.size else 0.0
    return bool(np.all(err <= bound)), ratio, bound
