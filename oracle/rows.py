"""Float64 scoring of many vocabulary rows at once (the C form of step.score), for loop replays.

Test infrastructure only (see the package docstring).  rows.c states the definition; it is the
one in step.py: m = max x, a = the first index at m, S = sum exp(x - m), c = 1/S, in float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rows.c")
LIB = os.path.join(HERE, "liboracle_rows.so")
CMD = ["gcc", "-O3", "-fPIC", "-shared", "-fopenmp", "-fno-math-errno", "-o", LIB, SRC, "-lmvec", "-lm"]

_lib = None


def build(verbose=False):
    """Compile rows.c in place (always recompiles)."""
    if verbose:
        print(" ".join(CMD), flush=True)
    subprocess.run(CMD, check=True)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        lib = ctypes.CDLL(LIB)
        lib.oracle_score_rows.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_score_rows.restype = ctypes.c_int64
        _lib = lib
    return _lib


def score_rows(x, dtype: str, threads: int = 0):
    """x: [n, V] (rows may be strided; elements of a row contiguous): uint16 bf16 bit patterns for
    "bf16", float32 for "fp32".  Returns (argmax int64 [n], conf float64 [n]).  Raises ValueError
    if a row holds a non-finite logit (a precondition of the step).  threads <= 0: OpenMP's default.
    The call releases the GIL (ctypes), so it can run beside other Python threads."""
    want = np.uint16 if dtype == "bf16" else np.float32
    x = np.asarray(x)
    if x.dtype != want:
        raise ValueError(f"{dtype} rows must be {np.dtype(want).name}, got {x.dtype}")
    if x.ndim != 2:
        raise ValueError("x must be [n, V]")
    n, V = x.shape
    a = np.empty(n, np.int64)
    c = np.empty(n, np.float64)
    if n == 0:
        return a, c
    if V > 1 and x.strides[1] != x.itemsize:
        raise ValueError("x must have contiguous rows")
    stride = x.strides[0] // x.itemsize
    bad = _load().oracle_score_rows(x.ctypes.data, 1 if dtype == "bf16" else 0, n, V, stride, a.ctypes.data,
                                    c.ctypes.data, int(threads))
    if bad < 0:
        raise MemoryError("oracle_score_rows: out of memory")
    if bad > 0:
        raise ValueError(f"{bad} of {n} rows hold non-finite logits")
    return a, c
