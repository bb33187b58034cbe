"""ctypes binding of libsaq.so (the C ABI declared in include/saq.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. torch supplies device memory and the current stream; nothing here
computes on tensors, and there is no fallback when the library is missing.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsaq.so")

SAQ_OK = 0
STATUS_NAMES = {
    0: "SAQ_OK", -1: "SAQ_ERR_NULL", -2: "SAQ_ERR_SHAPE", -3: "SAQ_ERR_UNSUPPORTED", -4: "SAQ_ERR_ALIGN",
    -5: "SAQ_ERR_RANGE", -6: "SAQ_ERR_WORKSPACE", -7: "SAQ_ERR_HIP", -8: "SAQ_ERR_NO_DEVICE", -9: "SAQ_ERR_ALIAS",
}

_lock = threading.Lock()
_lib = None

_vp, _i32, _f32, _f64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_double, ctypes.c_size_t

# (name, restype, argtypes) of every exported symbol
SIGNATURES = [
    ("saq_qknorm_rope", ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                       _f64, _f64, _vp]),
    ("saq_qknorm_rope_out", ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                           _i32, _i32, _f64, _f64, _vp]),
    ("saq_kept_blocks", _i32, [_f64, _i32]),
    ("saq_select_blocks_workspace_bytes", _sz, [_i32, _i32, _i32, _i32, _i32]),
    ("saq_select_blocks", ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _f64, _vp, _vp, _sz, _vp]),
    ("saq_select_blocks_noalloc", ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _f64, _vp, _vp]),
    ("saq_block_sparse_attn", ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _vp]),
    ("saq_qknorm_rope_pool", ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                            _i32, _i32, _f64, _f64, _i32, _vp, _sz, _vp]),
    ("saq_select_blocks_pooled", ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _f64, _vp, _vp, _sz, _vp]),
    ("saq_mask_overlap", ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    ("saq_pooled_change_out_len", _sz, []),
    ("saq_pooled_change", ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _sz, _vp]),
    ("saq_pooled_bytes", _sz, [_i32, _i32, _i32, _i32, _i32]),
    ("saq_reuse_state_len", _sz, []),
    ("saq_select_blocks_reuse", ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _f64, _f64, _i32, _vp, _vp, _sz, _vp,
                                               _sz, _vp, _sz, _vp]),
    ("saq_quantize_int8", ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    ("saq_dequantize_int8", ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp]),
    ("saq_quantize_fp8", ctypes.c_int, [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    ("saq_dequantize_fp8", ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp]),
    ("saq_block_sparse_attn_select", ctypes.c_int, [_vp, _vp, _vp, _vp, _sz, _i32, _i32, _i32, _i32, _i32, _f64,
                                                    _f32, _vp, _vp, _vp]),
    ("saq_status_string", ctypes.c_char_p, [ctypes.c_int]),
    ("saq_last_hip_error", ctypes.c_int, []),
]


class SaqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {STATUS_NAMES.get(status, status)} ({lib().saq_status_string(status).decode()})"
        if status == -7:
            msg += f", hipError {lib().saq_last_hip_error()}"
        super().__init__(msg)


def lib():
    """Load libsaq.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise ImportError(f"{LIB_PATH} is missing: build it with "
                                      "`python -m sparse_attention_qknorm_amd.build`")
                handle = ctypes.CDLL(LIB_PATH)
                for name, res, args in SIGNATURES:
                    fn = getattr(handle, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = handle
    return _lib


def check(status: int, where: str) -> None:
    if status != SAQ_OK:
        raise SaqError(status, where)
