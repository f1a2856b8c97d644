"""ctypes binding of libpa.so (see include/pa.h for the contract).

Argument marshalling only: tensors become raw device pointers and sizes, the
current torch stream becomes the hipStream_t.  Every step of the computation
runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa.so")

PA_OK = 0
PA_ERR_INVALID_ARGUMENT = 1
PA_ERR_NOT_IMPLEMENTED = 2
PA_ERR_WORKSPACE_TOO_SMALL = 3
PA_ERR_HIP = 4
PA_F16 = 0
PA_BF16 = 1
PROFILE_KINDS = ("scatter", "plan", "attention", "combine", "rotary")

EXPORTS = ("pa_scatter_kv", "pa_scatter_kv_paged", "pa_scatter_kv_fp8", "pa_scatter_kv_paged_fp8",
           "pa_rotary_scatter_kv",
           "pa_rotary_scatter_kv_fp8",
           "pa_seqlens_from_past",
           "pa_attention_workspace_size", "pa_attention", "pa_attention_rope",
           "pa_attention_noalloc",
           "pa_attention_fp8", "pa_attention_rope_fp8",
           "pa_validate_metadata", "pa_status_string", "pa_last_error",
           "pa_profile_enable", "pa_profile_select", "pa_profile_read")


class PAError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def lib():
    """Load libpa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m paged_kv_cache_pa_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                             ctypes.c_float, ctypes.c_size_t)
    L.pa_scatter_kv.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, vp]
    L.pa_scatter_kv.restype = i32
    L.pa_scatter_kv_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i64, i32, i32,
                                      i32, i32, vp]
    L.pa_scatter_kv_paged.restype = i32
    L.pa_scatter_kv_paged_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i64,
                                          i32, i32, i32, i32, vp]
    L.pa_scatter_kv_paged_fp8.restype = i32
    L.pa_scatter_kv_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, vp]
    L.pa_scatter_kv_fp8.restype = i32
    L.pa_rotary_scatter_kv.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                       i32, i64, i32, i64, i32, i32, i32, i32, i32, vp]
    L.pa_rotary_scatter_kv.restype = i32
    L.pa_rotary_scatter_kv_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp,
                                           vp, vp, vp, i32, i64, i32, i64, i32, i32, i32, i32,
                                           i32, vp]
    L.pa_rotary_scatter_kv_fp8.restype = i32
    L.pa_seqlens_from_past.argtypes = [vp, vp, vp, i32, vp]
    L.pa_seqlens_from_past.restype = i32
    L.pa_attention_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, i32]
    L.pa_attention_workspace_size.restype = sz
    L.pa_attention.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i64, f32, f32, i32,
                               i32, i32, i32, i32, i32, vp, sz, vp]
    L.pa_attention.restype = i32
    L.pa_attention_rope.argtypes = [vp, i64, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32,
                                    i64, i32, i64, f32, f32, i32, i32, i32, i32, i32, i32, vp, sz,
                                    vp]
    L.pa_attention_rope.restype = i32
    L.pa_attention_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i64, f32, f32,
                                       i32, i32, i32, i32, i32, i32, vp]
    L.pa_attention_noalloc.restype = i32
    L.pa_attention_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i64,
                                   f32, f32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    L.pa_attention_fp8.restype = i32
    L.pa_attention_rope_fp8.argtypes = [vp, i64, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                        vp, vp, i32, i64, i32, i32, i64, f32, f32, i32, i32, i32,
                                        i32, i32, i32, vp, sz, vp]
    L.pa_attention_rope_fp8.restype = i32
    L.pa_validate_metadata.argtypes = [vp, vp, vp, vp, i32, i64, i32, i64, i32,
                                       ctypes.POINTER(ctypes.c_uint32), vp]
    L.pa_validate_metadata.restype = i32
    L.pa_status_string.argtypes = [i32]
    L.pa_status_string.restype = ctypes.c_char_p
    L.pa_last_error.argtypes = []
    L.pa_last_error.restype = ctypes.c_char_p
    L.pa_profile_enable.argtypes = [i32]
    L.pa_profile_enable.restype = i32
    L.pa_profile_select.argtypes = [ctypes.c_uint32]
    L.pa_profile_select.restype = i32
    L.pa_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                  i32]
    L.pa_profile_read.restype = i32
    _lib = L
    return L


def check(status):
    if status != PA_OK:
        L = lib()
        raise PAError(status, f"{L.pa_status_string(status).decode()}: "
                              f"{L.pa_last_error().decode()}")
    return status
