"""Python binding of libr9k.so: block-scaled fp8 GEMMs on one MI355X (gfx950).

Argument marshalling only.  Every step of the path runs in the HIP kernels of
libr9k.so; this module takes torch tensors (device memory and streams are all
torch provides here), checks dtypes, allocates outputs and workspaces with
torch when the caller does not pass them, and calls the C ABI declared in
include/r9k.h under the same names.  There is no fallback: if the library is
not built, or a call returns an error, an exception is raised.

Tensor conventions (all contiguous, on the current CUDA/HIP device):
  bf16 values      torch.bfloat16 (or int16/uint16 holding the bits)
  fp8 e4m3 codes   torch.uint8 (or torch.float8_e4m3fn)
  scales, weights  torch.float32;  expert ids torch.int32
"""
from __future__ import annotations

import ctypes
import functools
import os
from ctypes import POINTER, c_char_p, c_int, c_int64, c_size_t, c_void_p

import torch

ABI_VERSION = 8
ENGINE_AUTO, ENGINE_SKINNY, ENGINE_TILED, ENGINE_SPLITK = 0, 1, 2, 3
TILE_AUTO, TILE_256X256, TILE_256X128, TILE_128X64, TILE_256X64 = 0, 1, 2, 3, 4

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libr9k.so")
_lib = None


class R9kError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: r9k error {code} ({strerror(code)})")


def lib() -> ctypes.CDLL:
    """Load libr9k.so (once).  Raises if it is missing or its ABI differs."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m block_scaled_fp8_r9k_amd.build` "
                              "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(LIB_PATH)
        L.r9k_abi_version.restype = c_int
        L.r9k_strerror.argtypes = [c_int]
        L.r9k_strerror.restype = c_char_p
        L.r9k_quant_act.argtypes = [c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_void_p]
        L.r9k_quant_weight.argtypes = [c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_void_p]
        L.r9k_encode_e4m3.argtypes = [c_void_p, c_int64, c_void_p, c_void_p]
        L.r9k_gemm_fp8_block_workspace.argtypes = [c_int64, c_int64, c_int64, POINTER(c_size_t)]
        L.r9k_gemm_fp8_block.argtypes = [c_void_p, c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_int64,
                                         c_void_p, c_void_p, c_size_t, c_void_p]
        L.r9k_gemm_fp8_block_qa.argtypes = [c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_int64, c_void_p,
                                            c_void_p, c_size_t, c_void_p]
        L.r9k_gemm_fp8_block_packed.argtypes = L.r9k_gemm_fp8_block.argtypes
        L.r9k_gemm_fp8_block_qa_packed.argtypes = L.r9k_gemm_fp8_block_qa.argtypes
        L.r9k_pack_weight.argtypes = [c_void_p, c_int64, c_int64, c_void_p, c_void_p]
        L.r9k_set_dispatch.argtypes = [c_int, c_int]
        L.r9k_set_tiled_plan.argtypes = [c_int, c_int]
        L.r9k_get_tiled_plan.argtypes = [POINTER(c_int), POINTER(c_int)]
        L.r9k_get_dispatch.argtypes = [POINTER(c_int), POINTER(c_int)]
        L.r9k_gemm_fp8_block_plan.argtypes = [c_int64, c_int64, c_int64, c_int, POINTER(c_int), POINTER(c_int)]
        L.r9k_moe_fp8_decode_workspace.argtypes = [c_int64] * 5 + [POINTER(c_size_t)]
        L.r9k_moe_ws_offset.argtypes = [c_int64] * 5 + [c_int, POINTER(c_size_t)]
        L.r9k_moe_fp8_decode.argtypes = [c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_int64, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_void_p, c_void_p,
                                         c_size_t, c_int, c_void_p]
        L.r9k_moe_fp8_decode_packed.argtypes = L.r9k_moe_fp8_decode.argtypes
        L.r9k_moe_fp8_decode_ex.argtypes = L.r9k_moe_fp8_decode.argtypes[:15] + [POINTER(MoeOpts), c_void_p]
        L.r9k_moe_route.argtypes = [c_void_p, c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p]
        L.r9k_gemm_fp8_block_bf16a.argtypes = [c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_int64, c_void_p,
                                               c_void_p]
        L.r9k_gemm_fp8_block_bf16a_packed.argtypes = L.r9k_gemm_fp8_block_bf16a.argtypes
        L.r9k_gemm_fp8_block_qa_noalloc.argtypes = [c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_int64,
                                                    c_void_p, c_int, c_void_p]
        v = L.r9k_abi_version()
        if v != ABI_VERSION:
            raise ImportError(f"libr9k.so has ABI version {v}, this binding needs {ABI_VERSION}")
        _lib = L
    return _lib


def abi_version() -> int:
    return lib().r9k_abi_version()


def strerror(code: int) -> str:
    return lib().r9k_strerror(code).decode()


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise R9kError(rc, what)


# torch's handle of the current stream as a plain integer: about 0.15 us a call,
# where torch.cuda.current_stream() builds a Stream object (about 2.7 us), which
# was the largest host cost of an eager call
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream) -> c_void_p:
    if stream is None:
        if _raw_stream is not None:
            return c_void_p(_raw_stream(torch.cuda.current_device()))
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t: torch.Tensor | None, dtypes, name: str) -> c_void_p:
    if t is None:
        return c_void_p(None)
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return c_void_p(t.data_ptr())


BF16 = (torch.bfloat16, torch.int16, torch.uint16)
FP8 = (torch.uint8, torch.float8_e4m3fn)
F32 = (torch.float32,)
I32 = (torch.int32,)


class Workspace:
    """A device workspace that grows on demand (each growth is a fresh
    allocation, zero-filled, though the library needs no initialisation: every
    call writes what it reads).  Not shared between streams that run
    concurrently."""

    def __init__(self, device=None):
        self.device = device
        self.buf: torch.Tensor | None = None

    def get(self, nbytes: int) -> torch.Tensor:
        nbytes = max(int(nbytes), 256)
        if self.buf is None or self.buf.numel() < nbytes:
            dev = self.device if self.device is not None else torch.device("cuda", torch.cuda.current_device())
            self.buf = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        return self.buf


_default_ws: dict[int, Workspace] = {}


def _workspace(ws: torch.Tensor | None, nbytes: int) -> torch.Tensor:
    if ws is not None:
        return ws
    dev = torch.cuda.current_device()
    if dev not in _default_ws:
        _default_ws[dev] = Workspace(torch.device("cuda", dev))
    return _default_ws[dev].get(nbytes)


# ------------------------------------------------------------------ quant ----

def quant_act(a: torch.Tensor, aq: torch.Tensor | None = None, as_: torch.Tensor | None = None, stream=None):
    """Per-token group-128 activation quant: a [M,K] bf16 -> (codes [M,K] u8, scales [M,K/128] f32)."""
    M, K = a.shape
    if aq is None:
        aq = torch.empty((M, K), dtype=torch.uint8, device=a.device)
    if as_ is None:
        as_ = torch.empty((M, K // 128 if K % 128 == 0 else 1), dtype=torch.float32, device=a.device)
    _check(lib().r9k_quant_act(_ptr(a, BF16, "a"), M, K, _ptr(aq, FP8, "aq"), _ptr(as_, F32, "as"),
                               _stream(stream)), "r9k_quant_act")
    return aq, as_


def quant_weight(w: torch.Tensor, wq: torch.Tensor | None = None, ws: torch.Tensor | None = None, stream=None):
    """128x128 block weight quant: w [N,K] bf16 -> (codes [N,K] u8, scales [N/128,K/128] f32)."""
    N, K = w.shape
    if wq is None:
        wq = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    if ws is None:
        ws = torch.empty((max(N // 128, 1), max(K // 128, 1)), dtype=torch.float32, device=w.device)
    _check(lib().r9k_quant_weight(_ptr(w, BF16, "w"), N, K, _ptr(wq, FP8, "wq"), _ptr(ws, F32, "ws"),
                                  _stream(stream)), "r9k_quant_weight")
    return wq, ws


def encode_e4m3(x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Elementwise fp32 -> e4m3fn codes with the library's device encoder."""
    n = x.numel()
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(lib().r9k_encode_e4m3(_ptr(x, F32, "x"), n, _ptr(out, FP8, "codes"), _stream(stream)),
           "r9k_encode_e4m3")
    return out


# ------------------------------------------------------------------- gemm ----

@functools.lru_cache(maxsize=4096)
def gemm_fp8_block_workspace(M: int, K: int, N: int) -> int:
    """Workspace bytes for a GEMM of this shape (r9k_gemm_fp8_block_workspace).  The answer depends on the
    shape (it covers every dispatch setting, and the library reads its tuning variables once) and on a
    forced tiled plan, which set_tiled_plan changes and then clears this cache; so it is cached: an eager
    call then pays no query."""
    b = c_size_t(0)
    _check(lib().r9k_gemm_fp8_block_workspace(M, K, N, ctypes.byref(b)), "r9k_gemm_fp8_block_workspace")
    return b.value


def gemm_fp8_block(aq, as_, w, ws, c=None, workspace=None, stream=None) -> torch.Tensor:
    """Block GEMM on pre-quantised activations (the split form) -> C [M,N] bf16."""
    M, K = aq.shape
    N = w.shape[0]
    if c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=aq.device)
    if M == 0:  # an empty batch: nothing to compute (an empty tensor has no device address to pass)
        return c
    nbytes = gemm_fp8_block_workspace(M, K, N)
    wsb = _workspace(workspace, nbytes)
    _check(lib().r9k_gemm_fp8_block(_ptr(aq, FP8, "aq"), _ptr(as_, F32, "as"), M, K, _ptr(w, FP8, "w"),
                                    _ptr(ws, F32, "ws"), N, _ptr(c, BF16, "c"), _ptr(wsb, FP8, "workspace"),
                                    wsb.numel(), _stream(stream)), "r9k_gemm_fp8_block")
    return c


def gemm_fp8_block_qa(a, w, ws, c=None, workspace=None, stream=None) -> torch.Tensor:
    """The fused form: bf16 activations quantised inside the GEMM -> C [M,N] bf16."""
    M, K = a.shape
    N = w.shape[0]
    if c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    if M == 0:  # an empty batch: nothing to compute (an empty tensor has no device address to pass)
        return c
    nbytes = gemm_fp8_block_workspace(M, K, N)
    wsb = _workspace(workspace, nbytes)
    _check(lib().r9k_gemm_fp8_block_qa(_ptr(a, BF16, "a"), M, K, _ptr(w, FP8, "w"), _ptr(ws, F32, "ws"), N,
                                       _ptr(c, BF16, "c"), _ptr(wsb, FP8, "workspace"), wsb.numel(),
                                       _stream(stream)), "r9k_gemm_fp8_block_qa")
    return c


NOALLOC_SCRATCH_BYTES = 64 << 20


def gemm_fp8_block_qa_noalloc(a, w, ws, c=None, packed: bool = False, stream=None) -> torch.Tensor:
    """The fused GEMM without a workspace (r9k_gemm_fp8_block_qa_noalloc): the library's own scratch on
    this GPU, no device allocation in the call (pass c to avoid torch's output allocation too).  Calls on
    one GPU must not overlap in time."""
    M, K = a.shape
    N = w.shape[0]
    if c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    if M == 0:  # an empty batch: nothing to compute (an empty tensor has no device address to pass)
        return c
    _check(lib().r9k_gemm_fp8_block_qa_noalloc(_ptr(a, BF16, "a"), M, K, _ptr(w, FP8, "w"), _ptr(ws, F32, "ws"), N,
                                               _ptr(c, BF16, "c"), 1 if packed else 0, _stream(stream)),
           "r9k_gemm_fp8_block_qa_noalloc")
    return c


def gemm_fp8_block_bf16a(a, w, ws, c=None, stream=None, packed: bool = False) -> torch.Tensor:
    """The bf16-activation variant at decode widths (M <= 16): a [M,K] bf16 (not quantised), w [N,K] fp8 codes
    (or their pack_weight copy when packed), ws [N/128,K/128] -> C [M,N] bf16."""
    M, K = a.shape
    N = w.shape[0]
    if c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    fn = lib().r9k_gemm_fp8_block_bf16a_packed if packed else lib().r9k_gemm_fp8_block_bf16a
    _check(fn(_ptr(a, BF16, "a"), M, K, _ptr(w, FP8, "w"), _ptr(ws, F32, "ws"), N, _ptr(c, BF16, "c"),
              _stream(stream)), "r9k_gemm_fp8_block_bf16a_packed" if packed else "r9k_gemm_fp8_block_bf16a")
    return c


def pack_weight(wq: torch.Tensor, wp: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Fragment-order copy of the weight codes (r9k_pack_weight): wq [N,K] u8
    row-major -> wp, also [N,K] u8 in shape, bytes in fragment order."""
    N, K = wq.shape
    if wp is None:
        wp = torch.empty((N, K), dtype=torch.uint8, device=wq.device)
    _check(lib().r9k_pack_weight(_ptr(wq, FP8, "wq"), N, K, _ptr(wp, FP8, "wp"), _stream(stream)),
           "r9k_pack_weight")
    return wp


def gemm_fp8_block_packed(aq, as_, wp, ws, c=None, workspace=None, stream=None) -> torch.Tensor:
    """gemm_fp8_block on fragment-order weights (pack_weight)."""
    M, K = aq.shape
    N = wp.shape[0]
    if c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=aq.device)
    if M == 0:  # an empty batch: nothing to compute (an empty tensor has no device address to pass)
        return c
    nbytes = gemm_fp8_block_workspace(M, K, N)
    wsb = _workspace(workspace, nbytes)
    _check(lib().r9k_gemm_fp8_block_packed(_ptr(aq, FP8, "aq"), _ptr(as_, F32, "as"), M, K, _ptr(wp, FP8, "wp"),
                                           _ptr(ws, F32, "ws"), N, _ptr(c, BF16, "c"),
                                           _ptr(wsb, FP8, "workspace"), wsb.numel(), _stream(stream)),
           "r9k_gemm_fp8_block_packed")
    return c


def gemm_fp8_block_qa_packed(a, wp, ws, c=None, workspace=None, stream=None) -> torch.Tensor:
    """gemm_fp8_block_qa on fragment-order weights (pack_weight)."""
    M, K = a.shape
    N = wp.shape[0]
    if c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    if M == 0:  # an empty batch: nothing to compute (an empty tensor has no device address to pass)
        return c
    nbytes = gemm_fp8_block_workspace(M, K, N)
    wsb = _workspace(workspace, nbytes)
    _check(lib().r9k_gemm_fp8_block_qa_packed(_ptr(a, BF16, "a"), M, K, _ptr(wp, FP8, "wp"), _ptr(ws, F32, "ws"),
                                              N, _ptr(c, BF16, "c"), _ptr(wsb, FP8, "workspace"), wsb.numel(),
                                              _stream(stream)), "r9k_gemm_fp8_block_qa_packed")
    return c


def set_dispatch(skinny_max_m: int = 255, engine: int = ENGINE_AUTO) -> None:
    _check(lib().r9k_set_dispatch(skinny_max_m, engine), "r9k_set_dispatch")


def set_tiled_plan(shape: int = TILE_AUTO, ksplit: int = 0) -> None:
    """Force the tiled engine's tile shape (TILE_*) and K split (0: the planner's) for later calls
    (r9k_set_tiled_plan).  A forced split changes the workspace a shape needs, so the cached
    workspace sizes are dropped."""
    _check(lib().r9k_set_tiled_plan(shape, ksplit), "r9k_set_tiled_plan")
    gemm_fp8_block_workspace.cache_clear()


def get_tiled_plan() -> tuple[int, int]:
    sh, ks = c_int(0), c_int(0)
    _check(lib().r9k_get_tiled_plan(ctypes.byref(sh), ctypes.byref(ks)), "r9k_get_tiled_plan")
    return sh.value, ks.value


def get_dispatch() -> tuple[int, int]:
    m, e = c_int(0), c_int(0)
    _check(lib().r9k_get_dispatch(ctypes.byref(m), ctypes.byref(e)), "r9k_get_dispatch")
    return m.value, e.value


KERNEL_NONE, KERNEL_DECODE, KERNEL_SKINNY, KERNEL_TILED, KERNEL_MID = 0, 1, 2, 3, 4


def gemm_fp8_block_plan(M: int, K: int, N: int, packed: bool = False) -> tuple[int, int]:
    """(kernel, ksplit) that a GEMM call of this shape runs (host only)."""
    k, s = c_int(0), c_int(0)
    _check(lib().r9k_gemm_fp8_block_plan(M, K, N, int(bool(packed)), ctypes.byref(k), ctypes.byref(s)),
           "r9k_gemm_fp8_block_plan")
    return k.value, s.value


# -------------------------------------------------------------------- moe ----

@functools.lru_cache(maxsize=1024)
def moe_fp8_decode_workspace(T: int, H: int, E: int, I: int, topk: int) -> int:
    b = c_size_t(0)
    _check(lib().r9k_moe_fp8_decode_workspace(T, H, E, I, topk, ctypes.byref(b)), "r9k_moe_fp8_decode_workspace")
    return b.value


def moe_ws_offset(T: int, H: int, E: int, I: int, topk: int, which: str) -> int:
    b = c_size_t(0)
    w = {"gu": 0, "h": 1, "y": 2, "hq": 3, "hs": 4}[which]
    _check(lib().r9k_moe_ws_offset(T, H, E, I, topk, w, ctypes.byref(b)), "r9k_moe_ws_offset")
    return b.value


class MoeOpts(ctypes.Structure):
    """r9k_moe_opts."""
    _fields_ = [("fused", c_int), ("packed", c_int), ("shared", c_void_p), ("shared_w", c_void_p)]


def moe_route(logits, topk: int, ids=None, w=None, stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """One-launch routing: logits [T,E] fp32 -> (topk ids [T,topk] int32, renormalised weights [T,topk] fp32)."""
    T, E = logits.shape
    if ids is None:
        ids = torch.empty((T, topk), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((T, topk), dtype=torch.float32, device=logits.device)
    _check(lib().r9k_moe_route(_ptr(logits, F32, "logits"), T, E, topk, _ptr(ids, I32, "ids"), _ptr(w, F32, "w"),
                               _stream(stream)), "r9k_moe_route")
    return ids, w


def moe_fp8_decode(x, topk_ids, topk_w, w13, w13_s, w2, w2_s, out=None, workspace=None, fused: bool = True,
                   stream=None, packed: bool = False, shared=None, shared_w=None) -> torch.Tensor:
    """Routed MoE decode: x [T,H] bf16, ids/weights [T,topk], experts w13 [E,2I,H], w2 [E,H,I] (fp8 +
    block scales) -> out [T,H] bf16.  packed: w13 and w2 are pack_weight copies (same shapes).
    shared [T,H] bf16 (and its per-token weight shared_w [T] fp32): the shared expert's output, added in the
    combine (r9k_moe_fp8_decode_ex)."""
    T, H = x.shape
    topk = topk_ids.shape[1]
    E, twoI, _ = w13.shape
    I = twoI // 2
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    nbytes = moe_fp8_decode_workspace(T, H, E, I, topk)
    wsb = _workspace(workspace, nbytes)
    if shared is not None or shared_w is not None:
        opts = MoeOpts(1 if fused else 0, 1 if packed else 0, _ptr(shared, BF16, "shared"),
                       _ptr(shared_w, F32, "shared_w"))
        _check(lib().r9k_moe_fp8_decode_ex(
            _ptr(x, BF16, "x"), T, H, _ptr(topk_ids, I32, "topk_ids"), _ptr(topk_w, F32, "topk_w"), topk,
            _ptr(w13, FP8, "w13"), _ptr(w13_s, F32, "w13_s"), _ptr(w2, FP8, "w2"), _ptr(w2_s, F32, "w2_s"), E, I,
            _ptr(out, BF16, "out"), _ptr(wsb, FP8, "workspace"), wsb.numel(), ctypes.byref(opts), _stream(stream)),
            "r9k_moe_fp8_decode_ex")
        return out
    fn = lib().r9k_moe_fp8_decode_packed if packed else lib().r9k_moe_fp8_decode
    _check(fn(_ptr(x, BF16, "x"), T, H, _ptr(topk_ids, I32, "topk_ids"), _ptr(topk_w, F32, "topk_w"), topk,
              _ptr(w13, FP8, "w13"), _ptr(w13_s, F32, "w13_s"), _ptr(w2, FP8, "w2"), _ptr(w2_s, F32, "w2_s"), E, I,
              _ptr(out, BF16, "out"), _ptr(wsb, FP8, "workspace"), wsb.numel(), 1 if fused else 0, _stream(stream)),
           "r9k_moe_fp8_decode_packed" if packed else "r9k_moe_fp8_decode")
    return out
