"""Attention KL-divergence oracle -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this package.  The product library never calls it.

Three independent CPU implementations live here:

* `streamkl_oracle.c` (built to `libstreamkl_oracle.so`, wrapped by `fwd` and
  `bwd` below): the fp64 definition of per-row KL(P1||P2), LSE1, LSE2 and the
  analytic gradients, one (batch, head) slice at a time.
* `reference_mp`: the same definition evaluated through probabilities in
  mpmath at high precision, for tiny shapes.
* `online`: the pages' coupled online recurrence over running
  (m1, l1, m2, l2, acc) and the split-K merge of those states, in fp64.

See the header of `streamkl_oracle.c` for the readings taken where the pages
are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "streamkl_oracle.c")
LIB_PATH = os.path.join(_HERE, "libstreamkl_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, no fast-math) and OpenMP."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def configure(lib):
    """Declare the C oracle's signatures on a loaded library and return it."""
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int64)
    i64, dbl, cint = ctypes.c_int64, ctypes.c_double, ctypes.c_int
    lib.skl_oracle_fwd.argtypes = [i64, i64, i64, dbl, cint, dp, dp, dp, dp, ip, i64, dp, dp, dp]
    lib.skl_oracle_fwd.restype = cint
    lib.skl_oracle_bwd.argtypes = [i64, i64, i64, dbl, cint, dp, dp, dp, dp, ip, i64, dp,
                                   dp, dp, dp, dp, dp, dp, dp]
    lib.skl_oracle_bwd.restype = cint
    lib.skl_oracle_threads.argtypes = []
    lib.skl_oracle_threads.restype = cint
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        _lib = configure(ctypes.CDLL(LIB_PATH))
    return _lib


def threads() -> int:
    """OpenMP threads the C oracle runs with."""
    return int(_load().skl_oracle_threads())


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):  # torch tensor
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _rows(nq: int, rows: Optional[Sequence[int]]) -> np.ndarray:
    if rows is None:
        return np.arange(nq, dtype=np.int64)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if r.size and (r.min() < 0 or r.max() >= nq):
        raise ValueError("row index out of range")
    return r


def fwd(q1, k1, q2, k2, scale: float, causal: bool, rows: Optional[Sequence[int]] = None):
    """Per-row (kl, lse1, lse2) for one (batch, head) slice; q*: [NQ,D], k*: [NK,D]."""
    q1, k1, q2, k2 = map(_f64, (q1, k1, q2, k2))
    nq, d = q1.shape
    nk = k1.shape[0]
    assert q2.shape == (nq, d) and k1.shape == (nk, d) and k2.shape == (nk, d)
    r = _rows(nq, rows)
    kl = np.empty(r.size)
    l1 = np.empty(r.size)
    l2 = np.empty(r.size)
    rc = _load().skl_oracle_fwd(nq, nk, d, float(scale), int(bool(causal)), _ptr(q1), _ptr(k1),
                                _ptr(q2), _ptr(k2), r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                r.size, _ptr(kl), _ptr(l1), _ptr(l2))
    if rc != 0:
        raise RuntimeError("oracle forward failed")
    return kl, l1, l2


def bwd(q1, k1, q2, k2, scale: float, causal: bool, g, rows: Optional[Sequence[int]] = None):
    """Gradients of L = sum_r g[r] * KL_{rows[r]} for one (batch, head) slice.

    Returns dict with kl, lse1, lse2 (per listed row), dq1, dq2 ([nrows, D]) and
    dk1, dk2 ([NK, D], contribution of the listed rows)."""
    q1, k1, q2, k2 = map(_f64, (q1, k1, q2, k2))
    nq, d = q1.shape
    nk = k1.shape[0]
    r = _rows(nq, rows)
    g = _f64(g).reshape(-1)
    assert g.size == r.size
    out = {k: np.empty(r.size) for k in ("kl", "lse1", "lse2")}
    out["dq1"] = np.empty((r.size, d))
    out["dq2"] = np.empty((r.size, d))
    out["dk1"] = np.empty((nk, d))
    out["dk2"] = np.empty((nk, d))
    rc = _load().skl_oracle_bwd(nq, nk, d, float(scale), int(bool(causal)), _ptr(q1), _ptr(k1),
                                _ptr(q2), _ptr(k2), r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                r.size, _ptr(g), _ptr(out["kl"]), _ptr(out["lse1"]), _ptr(out["lse2"]),
                                _ptr(out["dq1"]), _ptr(out["dq2"]), _ptr(out["dk1"]), _ptr(out["dk2"]))
    if rc != 0:
        raise RuntimeError("oracle backward failed")
    return out
