"""ctypes binding of libqlora.so (the C ABI declared in include/qlora.h).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind these entry points. Loading fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora.so")

QLORA_OK = 0
QLORA_EINVAL = -1
QLORA_EUNSUPPORTED = -2
QLORA_EWORKSPACE = -3
QLORA_EHIP = -4
QLORA_ENONFINITE = -5
NOALLOC_SCRATCH_BYTES = 64 << 20  # QLORA_NOALLOC_SCRATCH_BYTES

OP_FORWARD, OP_BACKWARD, OP_MLP_FORWARD, OP_MLP_BACKWARD = 0, 1, 2, 3
FMT_NF4, FMT_INT8, FMT_FP8 = 0, 1, 2
GRAD_BF16, GRAD_F32 = 0, 1

# Every function the header declares (checked by the CPU tests against include/qlora.h).
EXPORTS = [
    "qlora_quantize", "qlora_pack_codes", "qlora_dequantize", "qlora_workspace_size", "qlora_forward", "qlora_backward",
    "qlora_backward_noalloc", "swiglu_mlp_forward", "swiglu_mlp_backward", "swiglu_mlp_tiled_workspace_size", "swiglu_mlp_forward_tiled",
    "swiglu_mlp_backward_tiled", "qlora_rmsnorm_forward", "qlora_rmsnorm_backward", "qlora_rope_forward",
    "qlora_rope_backward", "qlora_rope_table", "qlora_forward_rope", "qlora_lmhead_prepare", "qlora_ce_workspace_size", "qlora_chunked_ce",
    "qlora_profile_begin", "qlora_profile_end",
    "qlora_status_string", "qlora_last_error",
]


class QLoraLayerC(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("absmax", ctypes.c_void_p),
        ("A", ctypes.c_void_p),
        ("B", ctypes.c_void_p),
        ("K", ctypes.c_int64),
        ("N", ctypes.c_int64),
        ("r", ctypes.c_int64),
        ("s", ctypes.c_float),
        ("format", ctypes.c_int32),
        ("grad_dtype", ctypes.c_int32),
    ]


class KernelTimeC(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


class QLoraError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


_lib = None


def lib():
    """Load libqlora.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} not found: build it with `python -m parameter_efficient_fine_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    LP = ctypes.POINTER(QLoraLayerC)
    L.qlora_quantize.argtypes = [ctypes.c_int, vp, i64, i64, vp, vp, vp, vp]
    L.qlora_pack_codes.argtypes = [ctypes.c_int, vp, vp, i64, i64, vp, vp, vp]
    L.qlora_dequantize.argtypes = [ctypes.c_int, vp, vp, i64, i64, vp, vp]
    L.qlora_workspace_size.argtypes = [ctypes.c_int, i64, i64, i64, i64]
    L.qlora_workspace_size.restype = sz
    L.qlora_forward.argtypes = [LP, vp, i64, vp, vp, vp, sz, vp]
    L.qlora_backward.argtypes = [LP, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp]
    L.qlora_backward_noalloc.argtypes = [LP, vp, vp, vp, i64, vp, vp, vp, vp]
    L.swiglu_mlp_forward.argtypes = [LP, LP, LP, vp, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    L.swiglu_mlp_backward.argtypes = [LP, LP, LP, vp, vp, vp, vp, vp, vp, i64, vp,
                                      ctypes.POINTER(vp), ctypes.POINTER(vp), vp, sz, vp]
    L.swiglu_mlp_tiled_workspace_size.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64]
    L.swiglu_mlp_tiled_workspace_size.restype = sz
    L.swiglu_mlp_forward_tiled.argtypes = [LP, LP, LP, vp, i64, i64, vp, vp, vp, sz, vp]
    L.swiglu_mlp_backward_tiled.argtypes = [LP, LP, LP, vp, vp, vp, i64, i64, vp, ctypes.POINTER(vp),
                                            ctypes.POINTER(vp), vp, sz, vp]
    ci, cf = ctypes.c_int, ctypes.c_float
    L.qlora_rmsnorm_forward.argtypes = [vp, vp, i64, i64, cf, vp, vp, vp]
    L.qlora_rmsnorm_backward.argtypes = [vp, vp, vp, vp, i64, i64, vp, vp]
    L.qlora_rope_forward.argtypes = [vp, vp, vp, i64, ci, ci, ci, cf, vp]
    L.qlora_rope_backward.argtypes = [vp, vp, vp, i64, ci, ci, ci, cf, vp]
    L.qlora_rope_table.argtypes = [ci, cf, i64, vp, vp]
    L.qlora_forward_rope.argtypes = [LP, vp, i64, vp, vp, i64, ci, vp, vp, vp]
    L.qlora_lmhead_prepare.argtypes = [vp, i64, i64, vp, vp, vp]
    L.qlora_ce_workspace_size.argtypes = [i64, i64, i64]
    L.qlora_ce_workspace_size.restype = sz
    L.qlora_chunked_ce.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, vp, vp, sz, vp]
    L.qlora_profile_begin.argtypes = [ctypes.c_int]
    L.qlora_profile_begin.restype = ctypes.c_int
    L.qlora_profile_end.argtypes = [ctypes.POINTER(KernelTimeC), ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    L.qlora_profile_end.restype = ctypes.c_int
    L.qlora_status_string.argtypes = [ctypes.c_int]
    L.qlora_status_string.restype = ctypes.c_char_p
    L.qlora_last_error.argtypes = []
    L.qlora_last_error.restype = ctypes.c_char_p
    for f in ("qlora_quantize", "qlora_pack_codes", "qlora_dequantize", "qlora_forward", "qlora_backward", "qlora_backward_noalloc",
              "swiglu_mlp_forward", "swiglu_mlp_backward", "swiglu_mlp_forward_tiled", "swiglu_mlp_backward_tiled", "qlora_rmsnorm_forward",
              "qlora_rmsnorm_backward", "qlora_rope_forward", "qlora_rope_backward", "qlora_rope_table",
              "qlora_forward_rope", "qlora_lmhead_prepare", "qlora_chunked_ce"):
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


def check(fn: str, status: int) -> None:
    if status != QLORA_OK:
        raise QLoraError(fn, status, lib().qlora_status_string(status).decode())
