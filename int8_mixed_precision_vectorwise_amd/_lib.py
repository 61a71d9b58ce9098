"""ctypes loader for libi8mp.so (no compute here: argument marshalling only)."""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libi8mp.so")

I8MP_OK = 0
I8MP_EINVAL = -1
I8MP_ERANGE = -2
I8MP_EWORKSPACE = -3
I8MP_EDEVICE = -4
I8MP_ELAUNCH = -5
I8MP_ESCRATCH = -6
I8MP_MAX_K = 133144
I8MP_NOALLOC_SCRATCH_BYTES = 32 << 20

# Every symbol include/i8mp.h declares.
EXPORTS = (
    "i8mp_status_string",
    "i8mp_abi_version",
    "i8mp_quant_workspace_bytes",
    "i8mp_int8_vectorwise_quant",
    "i8mp_outlier_extract",
    "i8mp_int8_linear_matmul",
    "i8mp_int8_mm_dequant",
    "i8mp_int8_vectorwise_dequant",
    "i8mp_linear_workspace_query",
    "i8mp_linear_quantize",
    "i8mp_linear_matmul_dequant",
    "i8mp_linear_forward",
    "i8mp_linear_forward_noalloc",
    "i8mp_colwise_quant_workspace_bytes",
    "i8mp_int8_colwise_quant",
    "i8mp_linear_backward_workspace_query",
    "i8mp_linear_backward",
    "i8mp_fp4_quantize",
    "i8mp_fp4_double_quant",
    "i8mp_fp4_dequantize",
    "i8mp_fp4_linear",
)


class LinearWorkspaceLayout(Structure):
    _fields_ = [
        ("bytes", c_size_t),
        ("q_offset", c_size_t),
        ("ldq", c_int64),
        ("absmax_offset", c_size_t),
        ("bitmap_offset", c_size_t),
        ("idx_offset", c_size_t),
        ("count_offset", c_size_t),
        ("xo_offset", c_size_t),
        ("cap_pad", c_int32),
        ("scratch_offset", c_size_t),
        ("scratch_bytes", c_size_t),
        ("idx_len", c_int64),
    ]


class BackwardWorkspaceLayout(Structure):
    _fields_ = [
        ("bytes", c_size_t),
        ("ld_n", c_int64),
        ("ld_m", c_int64),
        ("gq_offset", c_size_t),
        ("gs_offset", c_size_t),
        ("wtq_offset", c_size_t),
        ("wts_offset", c_size_t),
        ("gtq_offset", c_size_t),
        ("gts_offset", c_size_t),
        ("xtq_offset", c_size_t),
        ("xts_offset", c_size_t),
        ("scratch_offset", c_size_t),
        ("scratch_bytes", c_size_t),
    ]


class I8mpError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lib = None


def _declare(lib):
    lib.i8mp_status_string.argtypes = [c_int32]
    lib.i8mp_status_string.restype = c_char_p
    lib.i8mp_abi_version.argtypes = []
    lib.i8mp_abi_version.restype = c_int32
    lib.i8mp_quant_workspace_bytes.argtypes = [c_int64, c_int64]
    lib.i8mp_quant_workspace_bytes.restype = c_size_t
    lib.i8mp_int8_vectorwise_quant.argtypes = [c_void_p, c_int64, c_int64, c_int64, c_float, c_void_p,
                                               c_int64, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.i8mp_int8_vectorwise_quant.restype = c_int32
    lib.i8mp_outlier_extract.argtypes = [c_void_p, c_int64, c_int64, c_int64, c_void_p, c_int32, c_void_p,
                                         c_void_p, c_void_p, c_int64, c_void_p]
    lib.i8mp_outlier_extract.restype = c_int32
    lib.i8mp_int8_linear_matmul.argtypes = [c_void_p, c_int64, c_void_p, c_int64, c_int64, c_int64, c_int64,
                                            c_void_p, c_int64, c_void_p]
    lib.i8mp_int8_linear_matmul.restype = c_int32
    lib.i8mp_int8_mm_dequant.argtypes = [c_void_p, c_int64, c_void_p, c_void_p, c_void_p, c_int64, c_int64,
                                         c_void_p, c_int64, c_void_p, c_void_p, c_int32, c_void_p, c_int64,
                                         c_int64, c_void_p, c_int64, c_void_p]
    lib.i8mp_int8_mm_dequant.restype = c_int32
    lib.i8mp_int8_vectorwise_dequant.argtypes = [c_void_p, c_int64, c_int64, c_int64, c_void_p, c_int32, c_void_p,
                                                 c_int64, c_void_p]
    lib.i8mp_int8_vectorwise_dequant.restype = c_int32
    lib.i8mp_linear_workspace_query.argtypes = [c_int64, c_int64, c_int64, c_int32,
                                                POINTER(LinearWorkspaceLayout)]
    lib.i8mp_linear_workspace_query.restype = c_int32
    lib.i8mp_linear_forward.argtypes = [c_void_p, c_int64, c_int64, c_int64, c_void_p, c_int64, c_void_p,
                                        c_int64, c_void_p, c_float, c_int32, c_void_p, c_int64, c_void_p,
                                        c_size_t, c_void_p]
    lib.i8mp_linear_forward.restype = c_int32
    lib.i8mp_linear_forward_noalloc.argtypes = [c_void_p, c_int64, c_int64, c_int64, c_void_p, c_int64, c_void_p,
                                                c_int64, c_void_p, c_float, c_int32, c_void_p, c_int64, c_void_p]
    lib.i8mp_linear_forward_noalloc.restype = c_int32
    lib.i8mp_linear_quantize.argtypes = [c_void_p, c_int64, c_int64, c_int64, c_float, c_int32, c_void_p,
                                         c_size_t, c_void_p]
    lib.i8mp_linear_quantize.restype = c_int32
    lib.i8mp_linear_matmul_dequant.argtypes = [c_void_p, c_int64, c_void_p, c_size_t, c_int64, c_int64, c_int32,
                                               c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_void_p, c_int64,
                                               c_void_p]
    lib.i8mp_linear_matmul_dequant.restype = c_int32
    lib.i8mp_colwise_quant_workspace_bytes.argtypes = [c_int64, c_int64]
    lib.i8mp_colwise_quant_workspace_bytes.restype = c_size_t
    lib.i8mp_int8_colwise_quant.argtypes = [c_void_p, c_int64, c_int64, c_int64, c_void_p, c_void_p, c_int32,
                                            c_void_p, c_int64, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.i8mp_int8_colwise_quant.restype = c_int32
    lib.i8mp_linear_backward_workspace_query.argtypes = [c_int64, c_int64, c_int64, c_int32,
                                                         POINTER(BackwardWorkspaceLayout)]
    lib.i8mp_linear_backward_workspace_query.restype = c_int32
    lib.i8mp_linear_backward.argtypes = [c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64, c_int64,
                                         c_int64, c_int64, c_int32, c_void_p, c_size_t, c_void_p, c_int64,
                                         c_void_p, c_int64, c_void_p, c_size_t, c_void_p]
    lib.i8mp_linear_backward.restype = c_int32
    lib.i8mp_fp4_quantize.argtypes = [c_void_p, c_int64, c_int64, c_int64, c_void_p, c_int64, c_void_p, c_void_p]
    lib.i8mp_fp4_quantize.restype = c_int32
    lib.i8mp_fp4_double_quant.argtypes = [c_void_p, c_int64, c_void_p, c_void_p, c_void_p]
    lib.i8mp_fp4_double_quant.restype = c_int32
    lib.i8mp_fp4_dequantize.argtypes = [c_void_p, c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p, c_int32,
                                        c_void_p, c_int64, c_void_p]
    lib.i8mp_fp4_dequantize.restype = c_int32
    lib.i8mp_fp4_linear.argtypes = [c_void_p, c_int64, c_int64, c_int64, c_void_p, c_int64, c_void_p, c_void_p,
                                    c_void_p, c_int64, c_void_p, c_void_p, c_int64, c_void_p]
    lib.i8mp_fp4_linear.restype = c_int32


def lib():
    """The loaded library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m int8_mixed_precision_vectorwise_amd.build_lib` (there is no CPU fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        _declare(handle)
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    try:
        return lib().i8mp_status_string(status).decode()
    except RuntimeError:
        return "library not loaded"


def check(status: int, what: str) -> None:
    if status != I8MP_OK:
        raise I8mpError(status, what)
