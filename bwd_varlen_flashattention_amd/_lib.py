"""ctypes loader for libjfa.so and the C structs of include/jfa.h.

The library is built in-tree by ``bwd_varlen_flashattention_amd.build``.  There
is no fallback: if the library is missing or fails to load, importing the
binding raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# JFA_LIBRARY selects another in-tree build of the same sources (the race-hunting
# libjfa_debug_sync.so); by default the library is libjfa.so next to this file.
LIB_PATH = os.environ.get("JFA_LIBRARY") or os.path.join(_PKG, "libjfa.so")

JFA_OK = 0
JFA_ERR_INVALID_ARGUMENT = 1
JFA_ERR_UNSUPPORTED = 2
JFA_ERR_WORKSPACE_TOO_SMALL = 3
JFA_ERR_HIP = 4

# every symbol include/jfa.h declares
EXPORTS = (
    "jfa_fwd_workspace_size", "jfa_fwd", "jfa_bwd_workspace_size", "jfa_bwd",
    "jfa_decode_workspace_size", "jfa_decode_paged", "jfa_decode_paged_noalloc", "jfa_decode_num_splits",
    "jfa_status_string", "jfa_abi_version", "jfa_check_offsets", "jfa_check_paged_cache",
)
CHECK_OFFSETS_START, CHECK_OFFSETS_ORDER, CHECK_OFFSETS_END = 1, 2, 4
CHECK_SEQLEN_RANGE, CHECK_PAGE_RANGE = 8, 16
ABI_VERSION = 6
DECODE_SCRATCH_BYTES = 8 << 20   # JFA_DECODE_SCRATCH_BYTES
DECODE_COUNTER_BYTES = 256 << 10   # JFA_DECODE_COUNTER_BYTES


class KernelEventsStruct(ctypes.Structure):
    """jfa_kernel_events_t: caller-created hipEvent_t handles (or NULL)."""
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "fwd_start", "fwd_stop", "bwd_dq_start", "bwd_dq_stop",
        "bwd_dkdv_start", "bwd_dkdv_stop", "decode_start", "decode_stop")]


class AttnParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads_q", ctypes.c_int32),
        ("num_heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("total_k", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_k", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("broadcast_q", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("qkv_dtype", ctypes.c_int32),
        ("q_scale", ctypes.c_float),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("query_tile", ctypes.c_int32),
        ("events", ctypes.POINTER(KernelEventsStruct)),
    ]


class DecodeParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads_q", ctypes.c_int32),
        ("num_heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("q_len", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("q_dtype", ctypes.c_int32),
        ("q_scale", ctypes.c_float),
        ("single_launch", ctypes.c_int32),
        ("events", ctypes.POINTER(KernelEventsStruct)),
    ]


class JfaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed: {status_string(status)} ({status})")


_lib = None


def load() -> ctypes.CDLL:
    """Load libjfa.so once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m bwd_varlen_flashattention_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32p = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p
    ap, dp = ctypes.POINTER(AttnParams), ctypes.POINTER(DecodeParams)
    lib.jfa_fwd_workspace_size.argtypes = [ap]
    lib.jfa_fwd_workspace_size.restype = sz
    lib.jfa_fwd.argtypes = [ap, vp, vp, vp, i32p, i32p, vp, vp, vp, sz, vp]
    lib.jfa_fwd.restype = ctypes.c_int
    lib.jfa_bwd_workspace_size.argtypes = [ap]
    lib.jfa_bwd_workspace_size.restype = sz
    lib.jfa_bwd.argtypes = [ap, vp, vp, vp, vp, vp, vp, i32p, i32p, vp, vp, vp, vp, sz, vp]
    lib.jfa_bwd.restype = ctypes.c_int
    lib.jfa_decode_workspace_size.argtypes = [dp]
    lib.jfa_decode_workspace_size.restype = sz
    lib.jfa_decode_num_splits.argtypes = [dp]
    lib.jfa_decode_num_splits.restype = ctypes.c_int32
    lib.jfa_decode_paged.argtypes = [dp, vp, vp, vp, i32p, i32p, vp, vp, vp, sz, vp]
    lib.jfa_decode_paged.restype = ctypes.c_int
    lib.jfa_decode_paged_noalloc.argtypes = [dp, vp, vp, vp, i32p, i32p, vp, vp, vp]
    lib.jfa_decode_paged_noalloc.restype = ctypes.c_int
    lib.jfa_check_offsets.argtypes = [i32p, ctypes.c_int32, ctypes.c_int32, i32p, vp]
    lib.jfa_check_offsets.restype = ctypes.c_int
    lib.jfa_check_paged_cache.argtypes = [dp, i32p, i32p, i32p, vp]
    lib.jfa_check_paged_cache.restype = ctypes.c_int
    lib.jfa_status_string.argtypes = [ctypes.c_int]
    lib.jfa_status_string.restype = ctypes.c_char_p
    lib.jfa_abi_version.argtypes = []
    lib.jfa_abi_version.restype = ctypes.c_int
    if lib.jfa_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {lib.jfa_abi_version()}, the binding expects "
                          f"{ABI_VERSION}; rebuild it")
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().jfa_status_string(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != JFA_OK:
        raise JfaError(status, where)
