"""ctypes loader for libfp8mi.so, the C ABI declared in include/fp8mi.h.

The library must have been built in-tree (``python -m
fp8_precision_quantization_amd.build``); there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libfp8mi.so")
HEADER = os.path.join(ROOT, "include", "fp8mi.h")

FP8_OK = 0
FP8_ERR_INVALID_ARG = 1
FP8_ERR_UNSUPPORTED_SHAPE = 2
FP8_ERR_MISALIGNED = 3
FP8_ERR_UNSUPPORTED_DEVICE = 4
FP8_ERR_HIP = 5

FP8_E4M3, FP8_E5M2 = 0, 1
FP8_IN_F32, FP8_IN_BF16 = 0, 1
FP8_OUT_F32, FP8_OUT_BF16 = 0, 1
FP8_GRAN_TENSOR, FP8_GRAN_ROW, FP8_GRAN_BLOCK_1x128, FP8_GRAN_BLOCK_128x128 = 0, 1, 2, 3
FP8_SCALE_POW2 = 1
FP8_TRANSPOSE_OUT = 2
FP8_SPIKE_GUARD = 4
FP8_KV_E4M3, FP8_KV_E5M2, FP8_KV_BF16 = 0, 1, 2
FP8_KV_PER_TOKEN_HEAD, FP8_KV_PER_HEAD = 0, 1
FP8_GROUPED_MAX_TILES = 1983
HISTORY_BYTES = 128
DIAG_BYTES = 16
WORKSPACE_BYTES = 65536
MAX_TENSORS = 8

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_INT = ctypes.c_int
_U32 = ctypes.c_uint32


class Fp8Tensor(ctypes.Structure):
    """fp8_tensor, one descriptor of fp8_quantize_tensors (56 bytes)."""
    _fields_ = [("x", _P), ("rows", _I64), ("cols", _I64), ("q", _P), ("scale_inv", _P), ("amax", _P),
                ("diag", _P)]


# name -> (restype, argtypes); must match include/fp8mi.h
SIGNATURES = {
    "fp8_abi_version": (_INT, []),
    "fp8_status_string": (ctypes.c_char_p, [_INT]),
    "fp8_last_error": (ctypes.c_char_p, []),
    "fp8_workspace_size": (_I64, []),
    "fp8_history_init": (_INT, [_P, _I32, _P]),
    "fp8_history_set_guard": (_INT, [_P, ctypes.c_float, _P]),
    "fp8_amax": (_INT, [_P, _INT, _I64, _I64, _I64, _INT, _P, _P, _I64, _P]),
    "fp8_quantize": (_INT, [_P, _INT, _I64, _I64, _I64, _INT, _INT, _U32, _P, _P, _I64, _P, _P, _P, _P, _I64,
                            _P]),
    "fp8_quantize_noalloc": (_INT, [_P, _INT, _I64, _I64, _I64, _INT, _INT, _U32, _P, _P, _I64, _P, _P, _P,
                                    _P]),
    "fp8_quantize_dual": (_INT, [_P, _INT, _I64, _I64, _I64, _INT, _U32, _P, _P, _I64, _P, _I64, _P, _P, _P, _P,
                                 _I64, _P]),
    "fp8_quantize_tensors": (_INT, [_P, _I32, _INT, _INT, _U32, _P, _I64, _P]),
    "fp8_scaled_gemm": (_INT, [_P, _INT, _I64, _P, _INT, _I64, _I64, _I64, _I64, _P, _INT, _P, _INT,
                               _P, _INT, _I64, _P]),
    "fp8_blockscaled_gemm": (_INT, [_P, _I64, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _INT, _I64, _P]),
    "fp8_grouped_gemm": (_INT, [_P, _INT, _I64, _P, _INT, _I64, _I64, _I64, _I64, _I64, _I32, _P, _P, _INT,
                                _P, _INT, _P, _INT, _I64, _P, _I64, _P]),
    "fp8_kv_store": (_INT, [_P, _INT, _I64, _I64, _I32, _I32, _P, _INT, _INT, _U32, _P, _P, _I64, _P, _P]),
    "fp8_kv_load": (_INT, [_P, _INT, _INT, _P, _I64, _I32, _I32, _P, _I64, _INT, _P, _I64, _P]),
}


def header_functions() -> list:
    """Names of the functions include/fp8mi.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8_[a-z_0-9]+)\s*\(", text)))


class Fp8Error(RuntimeError):
    def __init__(self, status: int, func: str, message: str):
        self.status = status
        self.func = func
        super().__init__("%s -> %s: %s" % (func, status_name(status), message))


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libfp8mi.so is not built at %s; run `python -m fp8_precision_quantization_amd.build`"
                % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_name(status: int) -> str:
    return lib().fp8_status_string(status).decode()


def check(status: int, func: str):
    if status != FP8_OK:
        raise Fp8Error(status, func, lib().fp8_last_error().decode())
