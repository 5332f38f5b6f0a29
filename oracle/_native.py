"""ORACLE (test infrastructure only): builds and loads the oracle's C Jacobi.

The shared object goes to ``oracle/_build/`` (not tracked) and is rebuilt with
gcc whenever the source is newer.  Nothing on the HIP path loads it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "jacobi.c")
_OUT_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_OUT_DIR, "liboracle_jacobi.so")
_handle = None


def build(force: bool = False) -> str:
    os.makedirs(_OUT_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _handle
    if _handle is None:
        _handle = ctypes.CDLL(build())
        f = _handle.oracle_jacobi_eigh
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                      ctypes.c_int, ctypes.c_double]
    return _handle


def jacobi_raw(G: np.ndarray, max_sweeps: int = 60, tol: float = 1e-15):
    """Unsorted eigenpairs of symmetric G: (w, V) with G V = V diag(w)."""
    n = G.shape[0]
    A = np.array(G, dtype=np.float64, order="C", copy=True)
    Vt = np.empty((n, n), dtype=np.float64)
    w = np.empty(n, dtype=np.float64)
    sweeps = lib().oracle_jacobi_eigh(n, A.ctypes.data, Vt.ctypes.data, w.ctypes.data,
                                      max_sweeps, tol)
    return w, Vt.T.copy(), sweeps
