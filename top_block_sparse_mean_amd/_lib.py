"""ctypes view of libsparse_attn.so (the C ABI in include/sparse_attn.h).

The library is loaded from this package directory only; there is no fallback.
SPARSE_ATTN_LIB names another build of the same library to load instead (the tests
use it for a build whose host code carries address and undefined-behaviour checks);
it must exist too.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SPARSE_ATTN_LIB") or os.path.join(PKG, "libsparse_attn.so")

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_DEVICE = range(5)
SA_DTYPE_F32, SA_DTYPE_BF16 = 0, 1
SA_POOL_MEAN, SA_POOL_L2SUM = 0, 1
SA_SELECT_SUM, SA_SELECT_SOFTMAX, SA_SELECT_MAX, SA_SELECT_ATTN = 0, 1, 2, 3
SA_CHECK_SEQ, SA_CHECK_TABLE, SA_CHECK_PAGE, SA_CHECK_TOKEN = 1, 2, 4, 8

# Every symbol include/sparse_attn.h declares.
EXPORTS = ("sparse_attn_abi_version", "sparse_attn_status_string", "sparse_attn_last_error",
           "sparse_attn_validate", "sparse_attn_workspace_size", "sparse_attn_compress",
           "sparse_attn_compress_tail", "sparse_attn_append_kv", "sparse_attn_select", "sparse_attn_append_select",
           "sparse_attn_fwd", "sparse_attn_bucket_build", "sparse_attn_bucket_workspace_size", "sparse_attn_bucket_select",
           "sparse_attn_fwd_noalloc", "sparse_attn_decode_step", "sparse_attn_check_flags")


class SaParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("h_q", ctypes.c_int32),
        ("h_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_q", ctypes.c_int32),
        ("max_k", ctypes.c_int32),
        ("total_q", ctypes.c_int64),
        ("total_k", ctypes.c_int64),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("cu_seqlens_k", ctypes.c_void_p),
        ("q_pos0", ctypes.c_void_p),
        ("block", ctypes.c_int32),
        ("pool", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("topk_per_seq", ctypes.c_void_p),
        ("n_init", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("shared_selection", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("timing_events", ctypes.c_void_p * 2),
        ("block_table", ctypes.c_void_p),
        ("max_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("pool_overlap", ctypes.c_int32),
        ("select_mode", ctypes.c_int32),
        ("select_temperature", ctypes.c_float),
        ("attn_lse", ctypes.c_void_p),
    ]


class SaBucketIndex(ctypes.Structure):
    _fields_ = [
        ("block_tokens", ctypes.c_int32),
        ("count", ctypes.c_int32),
        ("cap_tokens", ctypes.c_int32),
        ("blocks_max", ctypes.c_int32),
        ("centroid", ctypes.c_void_p),
        ("member", ctypes.c_void_p),
        ("offset", ctypes.c_void_p),
        ("build_from", ctypes.c_int32),
    ]


class SparseAttnError(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__(f"{fn} failed: status {status} ({detail})")
        self.status = status
        self.detail = detail


_lib = None


def lib():
    """Load the built library; raise if it is not there (no CPU fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m top_block_sparse_mean_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(SaParams)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.sparse_attn_abi_version.restype = ctypes.c_int
        L.sparse_attn_abi_version.argtypes = []
        L.sparse_attn_last_error.argtypes = []
        L.sparse_attn_status_string.restype = ctypes.c_char_p
        L.sparse_attn_status_string.argtypes = [ctypes.c_int]
        L.sparse_attn_last_error.restype = ctypes.c_char_p
        L.sparse_attn_validate.argtypes = [P]
        L.sparse_attn_workspace_size.argtypes = [P, ctypes.POINTER(sz), ctypes.POINTER(sz)]
        L.sparse_attn_compress.argtypes = [P, vp, vp, vp]
        L.sparse_attn_compress_tail.argtypes = [P, ctypes.c_int32, vp, vp, vp]
        L.sparse_attn_select.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.sparse_attn_append_select.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.sparse_attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.sparse_attn_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        L.sparse_attn_append_kv.argtypes = [P, vp, vp, vp, vp, vp, vp]
        L.sparse_attn_decode_step.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        BX = ctypes.POINTER(SaBucketIndex)
        L.sparse_attn_bucket_build.argtypes = [P, vp, BX, vp]
        L.sparse_attn_bucket_workspace_size.argtypes = [P, BX, ctypes.c_int32, ctypes.POINTER(sz)]
        L.sparse_attn_bucket_select.argtypes = [P, vp, BX, ctypes.c_int32, vp, vp, vp, sz, vp]
        L.sparse_attn_check_flags.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int]
        for name in EXPORTS[3:]:
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def check(fn: str, status: int) -> None:
    if status != SA_OK:
        detail = lib().sparse_attn_last_error().decode()
        raise SparseAttnError(fn, status, detail)
