"""ctypes declarations of the C ABI in include/hsv.h (argument marshalling only)."""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhsv.so")

# hsv_status
HSV_OK = 0
HSV_ERR_NULL = 1
HSV_ERR_SHAPE = 2
HSV_ERR_UNSUPPORTED = 3
HSV_ERR_WORKSPACE = 4
HSV_ERR_DEVICE_CHECK = 5
HSV_ERR_HIP = 6

# hsv_dtype
HSV_F32 = 0
HSV_BF16 = 1

HSV_FLAG_VALIDATE = 1
HSV_FLAG_NO_PREFIX = 2
HSV_FLAG_NO_TREE = 4
HSV_FLAG_PHASE_PARTIALS = 8
HSV_FLAG_PHASE_MERGE = 16
HSV_FLAG_F32_PARTIALS = 32

HSV_NOALLOC_SCRATCH_BYTES = 32 << 20

# Every symbol include/hsv.h declares.
EXPORTS = (
    "hsv_verify_workspace_bytes",
    "hsv_verify_attn",
    "hsv_verify_attn_sparse",
    "hsv_verify_attn_paged",
    "hsv_verify_attn_sparse_paged",
    "hsv_verify_attn_noalloc",
    "hsv_tree_ancestor_mask",
    "hsv_gather_kv",
    "hsv_lse_merge",
    "hsv_select_kv_idx",
    "hsv_select_workspace_bytes",
    "hsv_tree_position_ids",
    "hsv_accept_path",
    "hsv_status_string",
    "hsv_version",
)


class HsvVerifyDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_draft", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("kv_capacity", ctypes.c_int32),
        ("max_ctx", ctypes.c_int32),
        ("n_sel", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("num_splits", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("block_size", ctypes.c_int32),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load libhsv.so from the package directory; fail loudly if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python long_context_tree_verify_amd/build_lib.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D = ctypes.POINTER(HsvVerifyDesc)
    lib.hsv_verify_workspace_bytes.argtypes = [D, ctypes.POINTER(sz)]
    lib.hsv_verify_attn.argtypes = [D, P, P, P, P, P, P, P, P, P, sz, P]
    lib.hsv_verify_attn_sparse.argtypes = [D, P, P, P, P, P, P, P, P, P, P, sz, P]
    lib.hsv_verify_attn_paged.argtypes = [D, P, P, P, P, i32, P, P, P, P, P, P, sz, P]
    lib.hsv_verify_attn_sparse_paged.argtypes = [D, P, P, P, P, i32, P, P, P, P, P, P, P, sz, P]
    lib.hsv_verify_attn_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, P]
    lib.hsv_tree_ancestor_mask.argtypes = [P, P, i32, i32, P]
    lib.hsv_gather_kv.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, P]
    lib.hsv_lse_merge.argtypes = [P, P, i32, i64, i32, P, P, i32, P]
    lib.hsv_select_kv_idx.argtypes = [P, P, i32, P, i32, i32, i32, i32, i32, i32, P, P, sz, P]
    lib.hsv_select_workspace_bytes.argtypes = [i32, i32, i32, ctypes.POINTER(sz)]
    lib.hsv_tree_position_ids.argtypes = [P, P, P, i32, i32, P]
    lib.hsv_accept_path.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, P]
    for name in ("hsv_verify_workspace_bytes", "hsv_verify_attn", "hsv_verify_attn_sparse",
                 "hsv_verify_attn_paged", "hsv_verify_attn_sparse_paged",
                 "hsv_verify_attn_noalloc", "hsv_tree_ancestor_mask", "hsv_gather_kv",
                 "hsv_lse_merge",
                 "hsv_select_kv_idx", "hsv_select_workspace_bytes", "hsv_tree_position_ids",
                 "hsv_accept_path"):
        getattr(lib, name).restype = ctypes.c_int
    lib.hsv_status_string.argtypes = [ctypes.c_int]
    lib.hsv_status_string.restype = ctypes.c_char_p
    lib.hsv_version.argtypes = []
    lib.hsv_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().hsv_status_string(code).decode()


class HsvError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)}")
