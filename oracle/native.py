"""Loader of the oracle's C part (exact_keys.c), built with the host C compiler.

Test infrastructure only, like the rest of oracle/.  The library is built
in-tree by the build step; if it is missing it is built here on first use.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "exact_keys.c")
LIB = os.path.join(HERE, "liboracle_keys.so")


def build() -> str:
    """Compile exact_keys.c into liboracle_keys.so (always)."""
    tmp = f"{LIB}.tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", tmp, SRC, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed on {SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        lib = ctypes.CDLL(LIB)
        lib.oracle_row_sumsq_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_row_sumsq_f32.restype = None
        _lib = lib
    return _lib


def row_sumsq_f32(A32: np.ndarray) -> np.ndarray:
    """Per row of a 2-D float32 array: the exact sum of squares rounded once to double."""
    A32 = np.ascontiguousarray(A32, dtype=np.float32)
    if A32.ndim != 2:
        raise ValueError("expected a 2-D array")
    rows, cols = A32.shape
    out = np.empty(rows, dtype=np.float64)
    if rows and cols:
        _load().oracle_row_sumsq_f32(A32.ctypes.data, rows, cols, out.ctypes.data)
    else:
        out[:] = 0.0
    return out
