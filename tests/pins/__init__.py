"""Independent re-derivations that pin the oracle (tests only); see pins.c."""
import ctypes
import os
import subprocess
from ctypes import POINTER, c_float, c_int, c_int64, c_uint8, c_uint16

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pins.c")
_LIB = os.path.join(_HERE, "libpins.so")
_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            tmp = _LIB + ".tmp%d" % os.getpid()
            subprocess.check_call(["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
                                   "-shared", "-pthread", "-o", tmp, _SRC, "-lm"])
            os.replace(tmp, _LIB)
        L = ctypes.CDLL(_LIB)
        L.pin_e4m3_encode_bits.argtypes = [c_float]
        L.pin_e4m3_encode_bits.restype = c_uint8
        L.pin_e4m3_encode_search.argtypes = [c_float]
        L.pin_e4m3_encode_search.restype = c_uint8
        L.pin_bf16_round_bits.argtypes = [c_float]
        L.pin_bf16_round_bits.restype = c_uint16
        for name, t in (("pin_e4m3_encode_bits_array", c_uint8), ("pin_e4m3_encode_search_array", c_uint8),
                        ("pin_bf16_round_bits_array", c_uint16)):
            getattr(L, name).argtypes = [POINTER(c_float), c_int64, POINTER(t), c_int]
        L.pin_div_correction_mismatches.argtypes = [c_int64, c_int64, c_int]
        L.pin_div_correction_mismatches.restype = c_int64
        L.pin_exhaustive.argtypes = [ctypes.c_void_p, c_int, c_int, POINTER(ctypes.c_uint32)]
        L.pin_exhaustive.restype = c_int64
        L.pin_scale_formula_mismatches.argtypes = []
        L.pin_scale_formula_mismatches.restype = c_int64
        _lib = L
    return _lib
