"""The C ABI on the host: the library loads, exports every symbol that
include/r9k.h declares, and every argument check returns its documented code
before touching a device.  No compute call runs here.
"""
import ctypes
import os
import re
from ctypes import c_int, c_int64, c_size_t, c_void_p

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "r9k.h")


@pytest.fixture(scope="module")
def L():
    import block_scaled_fp8_r9k_amd as r9k
    return r9k.lib()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(r9k_\w+)\s*\(", text, re.M)))


def _defines():
    text = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"#define\s+(R9K_\w+)\s+\(?(-?\d+)\)?", text)}


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 12, names
    for n in names:
        assert hasattr(L, n), f"libr9k.so does not export {n}"


def test_version_and_strerror(L):
    import block_scaled_fp8_r9k_amd as r9k
    d = _defines()
    assert L.r9k_abi_version() == d["R9K_ABI_VERSION"] == r9k.ABI_VERSION
    codes = [v for k, v in d.items() if k.startswith("R9K_ERR_") or k == "R9K_OK"]
    texts = {r9k.strerror(c) for c in codes}
    assert len(texts) == len(codes)                      # one distinct text per code
    assert "unknown" in r9k.strerror(-99)
    assert (r9k.ENGINE_AUTO, r9k.ENGINE_SKINNY, r9k.ENGINE_TILED) == (
        d["R9K_ENGINE_AUTO"], d["R9K_ENGINE_SKINNY"], d["R9K_ENGINE_TILED"])


A16 = c_void_p(0x10000)      # aligned fake addresses: never dereferenced by the checks below
B16 = c_void_p(0x20000)
C16 = c_void_p(0x30000)
ODD = c_void_p(0x10008)
NUL = c_void_p(None)
S = c_void_p(None)


def test_quant_checks(L):
    assert L.r9k_quant_act(NUL, 1, 128, B16, C16, S) == -1
    assert L.r9k_quant_act(A16, -1, 128, B16, C16, S) == -2
    assert L.r9k_quant_act(A16, 1, 100, B16, C16, S) == -2
    assert L.r9k_quant_act(A16, 1, 0, B16, C16, S) == -2
    assert L.r9k_quant_act(ODD, 1, 128, B16, C16, S) == -3
    assert L.r9k_quant_act(A16, 0, 128, B16, C16, S) == 0            # M == 0: nothing to do
    assert L.r9k_quant_weight(A16, 100, 128, B16, C16, S) == -2
    assert L.r9k_quant_weight(A16, 128, 128, NUL, C16, S) == -1
    assert L.r9k_quant_weight(A16, 128, 128, B16, ODD, S) == -3
    assert L.r9k_encode_e4m3(A16, -1, B16, S) == -2
    assert L.r9k_encode_e4m3(A16, 0, B16, S) == 0
    assert L.r9k_encode_e4m3(NUL, 4, B16, S) == -1


def _ws(L, M, K, N):
    b = c_size_t(0)
    rc = L.r9k_gemm_fp8_block_workspace(M, K, N, ctypes.byref(b))
    return rc, b.value


def _plan(L, M, K, N, packed=1):
    k, s = c_int(0), c_int(0)
    assert L.r9k_gemm_fp8_block_plan(M, K, N, packed, ctypes.byref(k), ctypes.byref(s)) == 0
    return k.value, s.value


def test_gemm_workspace_query(L):
    rc, b = _ws(L, 16, 4096, 14336)
    assert rc == 0 and b > 0 and b % 256 == 0
    rc, b4096 = _ws(L, 4096, 4096, 12288)
    assert rc == 0 and b4096 >= 4096 * 4096 + 4096 * 32 * 4      # room for A's codes and scales
    assert _ws(L, 16, 100, 128)[0] == -2
    assert _ws(L, 16, 128, 100)[0] == -2
    assert _ws(L, -1, 128, 128)[0] == -2
    assert L.r9k_gemm_fp8_block_workspace(1, 128, 128, None) == -1
    # an empty batch launches nothing and needs no workspace, for every shape (the query once divided
    # by the tiled engine's CTA count, which is zero here)
    for K, N in ((128, 128), (4096, 4096), (4096, 12288), (14336, 4096), (4096, 14336)):
        assert _ws(L, 0, K, N) == (0, 0)


def test_gemm_checks(L):
    big = 1 << 30
    f = L.r9k_gemm_fp8_block_qa
    assert f(NUL, 1, 128, B16, C16, 128, A16, B16, big, S) == -1
    assert f(A16, 1, 128, B16, C16, 128, A16, NUL, big, S) == -1
    assert f(A16, 1, 130, B16, C16, 128, A16, B16, big, S) == -2
    assert f(A16, 1, 128, B16, C16, 120, A16, B16, big, S) == -2
    assert f(ODD, 1, 128, B16, C16, 128, A16, B16, big, S) == -3
    assert f(A16, 0, 128, B16, C16, 128, A16, B16, 0, S) == 0        # M == 0
    assert f(A16, 1, 128, B16, C16, 128, A16, B16, 16, S) == -6      # workspace too small
    g = L.r9k_gemm_fp8_block
    assert g(A16, NUL, 1, 128, B16, C16, 128, A16, B16, big, S) == -1
    assert g(A16, B16, 1, 128, B16, C16, 128, ODD, B16, big, S) == -3
    assert g(A16, B16, 1, 128, B16, C16, 128, A16, B16, 0, S) == -6


def test_dispatch_settings(L):
    m, e = c_int(0), c_int(0)
    assert L.r9k_get_dispatch(ctypes.byref(m), ctypes.byref(e)) == 0
    old = (m.value, e.value)
    try:
        assert L.r9k_set_dispatch(-1, 0) == -2
        assert L.r9k_set_dispatch(255, 7) == -7 and L.r9k_set_dispatch(255, 4) == -7
        assert L.r9k_set_dispatch(255, 3) == 0                      # the split-K skinny kernel, forced
        assert L.r9k_set_dispatch(31, 2) == 0
        assert L.r9k_get_dispatch(ctypes.byref(m), ctypes.byref(e)) == 0
        assert (m.value, e.value) == (31, 2)
    finally:
        L.r9k_set_dispatch(*old)
    assert L.r9k_get_dispatch(None, ctypes.byref(e)) == -1


def test_tiled_plan_control(L):
    """r9k_set_tiled_plan forces the tiled engine's tile shape and K split; the plan query and the
    workspace query follow it (host only), and R9K_TILE_AUTO restores the planner's choice."""
    sh, ks = c_int(-1), c_int(-1)
    assert L.r9k_get_tiled_plan(ctypes.byref(sh), ctypes.byref(ks)) == 0
    old = (sh.value, ks.value)
    plan = lambda M, K, N: _plan(L, M, K, N)
    auto = plan(512, 4096, 4096)
    ws_auto = _ws(L, 512, 4096, 4096)[1]
    try:
        assert L.r9k_set_tiled_plan(5, 0) == -7 and L.r9k_set_tiled_plan(-1, 0) == -7
        assert L.r9k_set_tiled_plan(0, -1) == -7
        assert L.r9k_set_tiled_plan(2, 3) == 0                       # 256 x 128, split 3
        assert L.r9k_get_tiled_plan(ctypes.byref(sh), ctypes.byref(ks)) == 0 and (sh.value, ks.value) == (2, 3)
        assert plan(512, 4096, 4096) == (3, 3)
        assert plan(512, 256, 4096) == (3, 2)                        # the split clamped to K/128
        # the workspace follows: three fp32 partials of M x N beside the codes
        assert _ws(L, 512, 4096, 4096)[1] >= 3 * 4 * 512 * 4096
        assert L.r9k_set_tiled_plan(1, 4) == 0                       # 256 x 256 takes no split
        assert plan(512, 4096, 4096) == (3, 1)
    finally:
        assert L.r9k_set_tiled_plan(*old) == 0
    assert plan(512, 4096, 4096) == auto and _ws(L, 512, 4096, 4096)[1] == ws_auto
    assert L.r9k_get_tiled_plan(None, ctypes.byref(ks)) == -1


def test_moe_checks(L):
    b = c_size_t(0)
    assert L.r9k_moe_fp8_decode_workspace(16, 2048, 128, 768, 8, ctypes.byref(b)) == 0 and b.value > 0
    assert L.r9k_moe_fp8_decode_workspace(16, 2000, 128, 768, 8, ctypes.byref(b)) == -2
    assert L.r9k_moe_fp8_decode_workspace(16, 2048, 4, 768, 8, ctypes.byref(b)) == -2     # topk > E
    assert L.r9k_moe_fp8_decode_workspace(257, 2048, 128, 768, 8, ctypes.byref(b)) == -2
    off = c_size_t(0)
    for which in (0, 1, 2):
        assert L.r9k_moe_ws_offset(16, 2048, 128, 768, 8, which, ctypes.byref(off)) == 0
        assert off.value % 256 == 0 and off.value < b.value if which == 2 else True
    assert L.r9k_moe_ws_offset(16, 2048, 128, 768, 8, 9, ctypes.byref(off)) == -7
    big = 1 << 32
    args = [A16, 16, 2048, B16, C16, 8, A16, B16, C16, A16, 128, 768, B16, C16, big]
    f = L.r9k_moe_fp8_decode
    assert f(*args, 2, S) == -7                                         # fused must be 0 or 1
    bad = list(args); bad[0] = NUL
    assert f(*bad, 1, S) == -1
    bad = list(args); bad[3] = ODD
    assert f(*bad, 1, S) == -3
    bad = list(args); bad[-1] = 64
    assert f(*bad, 1, S) == -6
    bad = list(args); bad[1] = 0
    assert f(*bad, 1, S) == 0                                           # T == 0


def test_moe_route_and_ex_checks(L):
    import block_scaled_fp8_r9k_amd as r9k
    f = L.r9k_moe_route
    assert f(NUL, 16, 128, 8, B16, C16, S) == -1
    assert f(A16, 16, 128, 8, NUL, C16, S) == -1
    assert f(A16, 16, 128, 0, B16, C16, S) == -2                        # topk < 1
    assert f(A16, 16, 8, 9, B16, C16, S) == -2                          # topk > E
    assert f(A16, 16, 128, 65, B16, C16, S) == -2                       # topk > 64
    assert f(A16, 16, 0, 1, B16, C16, S) == -2                          # E < 1
    assert f(A16, -1, 128, 8, B16, C16, S) == -2
    assert f(ODD, 16, 128, 8, B16, C16, S) == -3
    assert f(A16, 0, 128, 8, B16, C16, S) == 0                          # T == 0: nothing to do
    big = 1 << 32
    args = [A16, 16, 2048, B16, C16, 8, A16, B16, C16, A16, 128, 768, B16, C16, big]
    g = L.r9k_moe_fp8_decode_ex
    assert g(*args, None, S) == -1                                      # no options
    o = r9k.MoeOpts(2, 0, None, None)
    assert g(*args, ctypes.byref(o), S) == -7                           # fused must be 0 or 1
    o = r9k.MoeOpts(1, 2, None, None)
    assert g(*args, ctypes.byref(o), S) == -7                           # packed must be 0 or 1
    o = r9k.MoeOpts(1, 0, None, 0x40000)
    assert g(*args, ctypes.byref(o), S) == -1                           # a weight without the shared term
    o = r9k.MoeOpts(1, 0, 0x40008, None)
    assert g(*args, ctypes.byref(o), S) == -3                           # misaligned shared output
    o = r9k.MoeOpts(1, 1, 0x40000, 0x50000)
    bad = list(args); bad[1] = 0
    assert g(*bad, ctypes.byref(o), S) == 0                             # T == 0


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.mark.skipif(_gpu_present(), reason="valid arguments would reach a real device")
def test_no_device_is_reported(L):
    """With valid arguments and no HIP device, every compute call returns -4."""
    big = 1 << 30
    assert L.r9k_quant_act(A16, 1, 128, B16, C16, S) == -4
    assert L.r9k_quant_weight(A16, 128, 128, B16, C16, S) == -4
    assert L.r9k_encode_e4m3(A16, 4, B16, S) == -4
    assert L.r9k_gemm_fp8_block_qa(A16, 1, 128, B16, C16, 128, A16, B16, big, S) == -4
    assert L.r9k_gemm_fp8_block(A16, B16, 1, 128, B16, C16, 128, A16, B16, big, S) == -4
    assert L.r9k_moe_fp8_decode(A16, 16, 2048, B16, C16, 8, A16, B16, C16, A16, 128, 768, B16, C16,
                                1 << 32, 1, S) == -4


def test_binding_refuses_host_tensors():
    import torch
    import block_scaled_fp8_r9k_amd as r9k
    with pytest.raises(ValueError):
        r9k.quant_act(torch.zeros((1, 128), dtype=torch.bfloat16))


def test_noalloc_checks(L):
    # the allocation-free entry point's host checks, before any device is touched
    f = L.r9k_gemm_fp8_block_qa_noalloc
    assert f(NUL, 1, 128, B16, C16, 128, A16, 0, S) == -1
    assert f(A16, 1, 130, B16, C16, 128, A16, 0, S) == -2
    assert f(A16, 1, 128, B16, C16, 128, A16, 2, S) == -7
    assert f(ODD, 1, 128, B16, C16, 128, A16, 0, S) == -3
    assert f(A16, 0, 128, B16, C16, 128, A16, 0, S) == 0           # M == 0: nothing to do
    d = _defines()
    assert "R9K_NOALLOC_SCRATCH_BYTES" not in d or d["R9K_NOALLOC_SCRATCH_BYTES"] > 0
    rc, need = _ws(L, 8192, 8192, 1024)
    assert rc == 0 and need > 64 << 20                             # beyond the scratch: refused
    assert f(A16, 8192, 8192, B16, C16, 1024, A16, 0, S) == -6
