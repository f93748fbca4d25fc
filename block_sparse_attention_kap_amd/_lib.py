"""ctypes declarations of the libcosa C ABI (include/cosa.h)."""
from __future__ import annotations

import ctypes
import os

COSA_OK, COSA_ERR_INVALID_ARG, COSA_ERR_UNSUPPORTED, COSA_ERR_HIP, COSA_ERR_SCRATCH = 0, -1, -2, -3, -4
COSA_NOALLOC_SCRATCH_MIB = 128
COSA_F32, COSA_BF16 = 0, 1
COSA_MAX_VARLEN_BATCH = 128
CAP_COMPUTED, CAP_VISITED = 0, 1
SKIP_OFF, SKIP_MAXDIFF, SKIP_MASS = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

# every symbol include/cosa.h declares
EXPORTS = ["cosa_list_capacity", "cosa_kap_workspace_bytes", "cosa_proxy_select",
           "cosa_proxy_select_noalloc",
           "cosa_ordered_sparse_attn", "cosa_prefill", "cosa_dense_attn", "cosa_status_string",
           "cosa_version"]


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int), ("q_heads", ctypes.c_int), ("kv_heads", ctypes.c_int),
                ("seq_len", ctypes.c_int), ("head_dim", ctypes.c_int), ("block", ctypes.c_int),
                ("causal", ctypes.c_int), ("scale", ctypes.c_float), ("dtype", ctypes.c_int),
                ("seq_lens", ctypes.POINTER(ctypes.c_int32))]


class KapParams(ctypes.Structure):
    _fields_ = [("budget", ctypes.c_double), ("pool", ctypes.c_int), ("pool_mode", ctypes.c_int),
                ("agg_mode", ctypes.c_int), ("sel_mode", ctypes.c_int), ("mass", ctypes.c_double),
                ("force_sink", ctypes.c_int), ("force_diag", ctypes.c_int),
                ("order_mode", ctypes.c_int), ("share_kv", ctypes.c_int)]


class OskParams(ctypes.Structure):
    _fields_ = [("tight_budget", ctypes.c_double), ("cap_mode", ctypes.c_int),
                ("skip_mode", ctypes.c_int), ("skip_param", ctypes.c_float),
                ("vote_rows", ctypes.c_int), ("shared_lists", ctypes.c_int)]


class CosaError(RuntimeError):
    def __init__(self, status: int, msg: str = ""):
        self.status = status
        super().__init__(f"libcosa status {status}: {msg}")


def lib_path() -> str:
    return os.environ.get("COSA_LIB", os.path.join(_HERE, "libcosa.so"))


def lib():
    """Load libcosa.so (raises if it was not built)."""
    global _LIB
    if _LIB is None:
        p = lib_path()
        if not os.path.exists(p):
            raise ImportError(f"{p} not found: build it with __graft_entry__.build() "
                              "(there is no CPU fallback)")
        L = ctypes.CDLL(p)
        vp, ip, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        sp, kp, op = ctypes.POINTER(Shape), ctypes.POINTER(KapParams), ctypes.POINTER(OskParams)
        L.cosa_list_capacity.argtypes = [sp, ctypes.c_double]
        L.cosa_list_capacity.restype = ip
        L.cosa_kap_workspace_bytes.argtypes = [sp, kp]
        L.cosa_kap_workspace_bytes.restype = sz
        L.cosa_proxy_select.argtypes = [sp, kp, vp, vp, vp, sz, vp, vp, vp, vp, ip, vp]
        L.cosa_proxy_select.restype = ip
        L.cosa_proxy_select_noalloc.argtypes = [sp, kp, vp, vp, vp, vp, vp, vp, ip, vp]
        L.cosa_proxy_select_noalloc.restype = ip
        L.cosa_ordered_sparse_attn.argtypes = [sp, op, vp, vp, vp, vp, vp, ip, vp, vp, vp, vp, vp, vp]
        L.cosa_ordered_sparse_attn.restype = ip
        L.cosa_prefill.argtypes = [sp, kp, op, vp, vp, vp, vp, sz, vp, vp, vp, ip, vp, vp, ip,
                                   vp, vp, vp]
        L.cosa_prefill.restype = ip
        L.cosa_dense_attn.argtypes = [sp, vp, vp, vp, vp, vp, vp]
        L.cosa_dense_attn.restype = ip
        L.cosa_status_string.argtypes = [ip]
        L.cosa_status_string.restype = ctypes.c_char_p
        L.cosa_version.argtypes = []
        L.cosa_version.restype = ip
        _LIB = L
    return _LIB


def check(status: int) -> None:
    if status < 0:
        raise CosaError(status, lib().cosa_status_string(status).decode())
