"""ctypes view of libgdn (include/gdn.h).  Loading fails loudly when the built
library is missing: there is no fallback implementation."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")

ABI_VERSION = 4  # GDN_ABI_VERSION of include/gdn.h this binding matches
GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_EWORKSPACE, GDN_EHIP = 0, -1, -2, -3, -4
GDN_DTYPE_BF16, GDN_DTYPE_F32 = 0, 1
CP_MODES = {"off": 0, "exact": 1, "warmup": 2, "auto": 3}
CP_NAMES = {v: k for k, v in CP_MODES.items()}

# Every exported entry point of include/gdn.h.
EXPORTS = ("gdn_abi_version", "gdn_status_str", "gdn_last_error", "gdn_fwd_plan", "gdn_fwd", "gdn_fwd_noalloc",
           "gdn_chunk_cumsum", "gdn_bwd_plan", "gdn_bwd")
NOALLOC_SCRATCH_BYTES = 64 << 20  # GDN_NOALLOC_SCRATCH_BYTES of include/gdn.h


class FwdDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("T", ctypes.c_int64),
        ("H_qk", ctypes.c_int32), ("H_v", ctypes.c_int32),
        ("K", ctypes.c_int32), ("V", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32),
        ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int32)),
        ("scale", ctypes.c_float),
        ("has_h0", ctypes.c_int32), ("want_ht", ctypes.c_int32),
        ("o_dtype", ctypes.c_int32), ("chunk", ctypes.c_int32),
        ("cp_mode", ctypes.c_int32), ("cp_lambda", ctypes.c_float),
        ("cp_segment_chunks", ctypes.c_int32), ("cp_warmup_chunks", ctypes.c_int32),
    ]


class FwdPlanInfo(ctypes.Structure):
    _fields_ = [
        ("workspace_bytes", ctypes.c_size_t),
        ("total_chunks", ctypes.c_int32), ("segment_chunks", ctypes.c_int32),
        ("num_segments", ctypes.c_int32), ("warmup_chunks", ctypes.c_int32),
        ("cp_mode", ctypes.c_int32), ("workgroups", ctypes.c_int32),
    ]


class FwdPtrs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p),
        ("initial_state", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("final_state", ctypes.c_void_p),
        ("h", ctypes.c_void_p), ("A", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
    ]


class BwdDesc(ctypes.Structure):
    _fields_ = [
        ("fwd", FwdDesc),
        ("has_dht", ctypes.c_int32), ("grad_dtype", ctypes.c_int32), ("saved_fwd", ctypes.c_int32),
    ]


class BwdPlanInfo(ctypes.Structure):
    _fields_ = [
        ("workspace_bytes", ctypes.c_size_t),
        ("total_chunks", ctypes.c_int32), ("segment_chunks", ctypes.c_int32),
        ("num_segments", ctypes.c_int32), ("warmup_chunks", ctypes.c_int32),
        ("cp_mode", ctypes.c_int32), ("workgroups_reverse", ctypes.c_int32),
        ("workgroups_local", ctypes.c_int32),
    ]


class BwdPtrs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p),
        ("initial_state", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
        ("dO", ctypes.c_void_p), ("d_final_state", ctypes.c_void_p),
        ("h", ctypes.c_void_p), ("A", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("dg", ctypes.c_void_p), ("dbeta", ctypes.c_void_p),
        ("d_initial_state", ctypes.c_void_p),
    ]


_lib = None


def lib():
    """The loaded library (RuntimeError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libgdn.so not found at {LIB_PATH}; build it with "
                               "`python -m gated_deltanet_chunked_chunk_amd.build` or __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.gdn_abi_version.restype = ctypes.c_int
        L.gdn_abi_version.argtypes = []
        L.gdn_status_str.restype = ctypes.c_char_p
        L.gdn_status_str.argtypes = [ctypes.c_int]
        L.gdn_last_error.restype = ctypes.c_char_p
        L.gdn_last_error.argtypes = []
        L.gdn_fwd_plan.restype = ctypes.c_int
        L.gdn_fwd_plan.argtypes = [ctypes.POINTER(FwdDesc), ctypes.POINTER(FwdPlanInfo)]
        L.gdn_fwd.restype = ctypes.c_int
        L.gdn_fwd.argtypes = [ctypes.POINTER(FwdDesc), ctypes.POINTER(FwdPtrs), ctypes.c_void_p, ctypes.c_size_t,
                              ctypes.c_void_p]
        L.gdn_fwd_noalloc.restype = ctypes.c_int
        L.gdn_fwd_noalloc.argtypes = [ctypes.POINTER(FwdDesc), ctypes.POINTER(FwdPtrs), ctypes.c_void_p]
        if L.gdn_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.gdn_abi_version()}, this binding expects "
                               f"{ABI_VERSION}; rebuild it")
        L.gdn_chunk_cumsum.restype = ctypes.c_int
        L.gdn_chunk_cumsum.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_void_p]
        L.gdn_bwd_plan.restype = ctypes.c_int
        L.gdn_bwd_plan.argtypes = [ctypes.POINTER(BwdDesc), ctypes.POINTER(BwdPlanInfo)]
        L.gdn_bwd.restype = ctypes.c_int
        L.gdn_bwd.argtypes = [ctypes.POINTER(BwdDesc), ctypes.POINTER(BwdPtrs), ctypes.c_void_p, ctypes.c_size_t,
                              ctypes.c_void_p]
        _lib = L
    return _lib


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{lib().gdn_status_str(status).decode()}: {message}")
        self.status = status


def check(status: int) -> None:
    if status == GDN_OK:
        return
    msg = lib().gdn_last_error().decode()
    if status in (GDN_EINVAL, GDN_EUNSUPPORTED):
        raise ValueError(f"{lib().gdn_status_str(status).decode()}: {msg}")
    raise GdnError(status, msg)
