"""ctypes view of the C ABI declared in include/streamkl.h.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libstreamkl.so.  Loading fails loudly if the library has not been
built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libstreamkl.so")

STREAMKL_OK = 0
STREAMKL_ERR_NULL = 1
STREAMKL_ERR_SHAPE = 2
STREAMKL_ERR_DTYPE = 3
STREAMKL_ERR_ALIGN = 4
STREAMKL_ERR_WORKSPACE = 5
STREAMKL_ERR_HIP = 6

STREAMKL_BF16 = 0
STREAMKL_FP32 = 1
STREAMKL_FP8_E4M3 = 2

NOALLOC_SCRATCH_BYTES = 64 << 20  # STREAMKL_NOALLOC_SCRATCH_BYTES

# Every function include/streamkl.h declares, in declaration order.
EXPORTS = (
    "streamkl_fwd",
    "streamkl_fwd_splitk_workspace_size",
    "streamkl_fwd_splitk",
    "streamkl_fwd_splitk_noalloc",
    "streamkl_bwd_workspace_size",
    "streamkl_bwd_workspace_size_min",
    "streamkl_bwd",
    "streamkl_bwd_prepare",
    "streamkl_bwd_dk",
    "streamkl_bwd_dq",
    "streamkl_fwd_varlen",
    "streamkl_bwd_varlen_workspace_size",
    "streamkl_bwd_varlen",
    "streamkl_status_string",
    "streamkl_version",
    "streamkl_probe_mfma_bf16",
)


class Problem(ctypes.Structure):
    """Mirror of streamkl_problem."""
    _fields_ = [
        ("B", ctypes.c_int64),
        ("H", ctypes.c_int64),
        ("NQ", ctypes.c_int64),
        ("NK", ctypes.c_int64),
        ("D", ctypes.c_int64),
        ("scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class VarlenProblem(ctypes.Structure):
    """Mirror of streamkl_varlen_problem (offset arrays are host pointers)."""
    _fields_ = [
        ("B", ctypes.c_int64),
        ("H", ctypes.c_int64),
        ("D", ctypes.c_int64),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("cu_seqlens_k", ctypes.c_void_p),
        ("scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class StreamKLError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libstreamkl.so (built by attention_kl_divergence_online_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m attention_kl_divergence_online_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        pp = ctypes.POINTER(Problem)
        L.streamkl_fwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.streamkl_fwd.restype = ctypes.c_int
        L.streamkl_fwd_splitk_workspace_size.argtypes = [pp, ctypes.c_int]
        L.streamkl_fwd_splitk_workspace_size.restype = sz
        L.streamkl_fwd_splitk.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp, sz, vp]
        L.streamkl_fwd_splitk.restype = ctypes.c_int
        L.streamkl_fwd_splitk_noalloc.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp]
        L.streamkl_fwd_splitk_noalloc.restype = ctypes.c_int
        L.streamkl_bwd_workspace_size.argtypes = [pp]
        L.streamkl_bwd_workspace_size.restype = sz
        L.streamkl_bwd_workspace_size_min.argtypes = [pp]
        L.streamkl_bwd_workspace_size_min.restype = sz
        L.streamkl_bwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.streamkl_bwd.restype = ctypes.c_int
        L.streamkl_bwd_prepare.argtypes = [pp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.streamkl_bwd_prepare.restype = ctypes.c_int
        for name in ("streamkl_bwd_dk", "streamkl_bwd_dq"):
            fn = getattr(L, name)
            fn.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
            fn.restype = ctypes.c_int
        vpp = ctypes.POINTER(VarlenProblem)
        L.streamkl_fwd_varlen.argtypes = [vpp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.streamkl_fwd_varlen.restype = ctypes.c_int
        L.streamkl_bwd_varlen_workspace_size.argtypes = [vpp]
        L.streamkl_bwd_varlen_workspace_size.restype = sz
        L.streamkl_bwd_varlen.argtypes = [vpp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.streamkl_bwd_varlen.restype = ctypes.c_int
        L.streamkl_status_string.argtypes = [ctypes.c_int]
        L.streamkl_status_string.restype = ctypes.c_char_p
        L.streamkl_version.argtypes = []
        L.streamkl_version.restype = ctypes.c_int
        L.streamkl_probe_mfma_bf16.argtypes = [ctypes.c_int64, ctypes.c_int64, vp, vp]
        L.streamkl_probe_mfma_bf16.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().streamkl_status_string(int(status)).decode()


def check(status: int, what: str) -> None:
    if status != STREAMKL_OK:
        raise StreamKLError(status, what)
