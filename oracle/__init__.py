"""CPU oracle for row-wise top-k selection -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The library under test never
does, and it shares no code with it.

The oracle is ``oracle.c``: a per-row full sort under the strict total order
"larger value first; +0 before -0; lower index first among equal values",
taking the first k (see the header of ``oracle.c`` for the readings).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, BAD_ARG, NAN, NOMEM = 0, 1, 4, 6
_DT = {"bf16": 0, "f32": 1}

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain C, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.oracle_topk.restype = ctypes.c_int
        lib.oracle_topk.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int32, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_topk_lengths.restype = ctypes.c_int
        lib.oracle_topk_lengths.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_sample.restype = ctypes.c_int
        lib.oracle_sample.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return _load().oracle_max_threads()


def topk(raw: np.ndarray, dtype: str, n: int, k: int, sorted_index=True,
         return_value: bool = True, nthreads: int = 1
         ) -> Tuple[int, np.ndarray, Optional[np.ndarray]]:
    """Top-k of each row of ``raw`` ([batch, row_stride] raw element bits:
    uint16 for bf16, float32 for fp32).  ``sorted_index``: 0/False any
    order, 1/True ascending index, 2 by value (largest first).  Returns
    (status, indices int32 [batch, k], values [batch, k] of raw's dtype or
    None)."""
    lib = _load()
    raw = np.ascontiguousarray(raw)
    want = np.uint16 if dtype == "bf16" else np.float32
    if raw.dtype != want:
        raise TypeError("raw must be %s for %s" % (np.dtype(want).name, dtype))
    batch, row_stride = raw.shape
    idx = np.zeros((batch, k), dtype=np.int32)
    val = np.zeros((batch, k), dtype=want) if return_value else None
    st = lib.oracle_topk(raw.ctypes.data, _DT[dtype], batch, n, row_stride, k,
                         int(sorted_index), int(bool(return_value)), idx.ctypes.data,
                         val.ctypes.data if val is not None else None, int(nthreads))
    return st, idx, val


def topk_lengths(raw: np.ndarray, dtype: str, n: int, k: int, lengths, sorted_index=True,
                 return_value: bool = True, nthreads: int = 1
                 ) -> Tuple[int, np.ndarray, Optional[np.ndarray]]:
    """As topk(), with row r's valid columns [0, lengths[r]) (clamped to
    [0, n]); the other columns act as -inf and are never read."""
    lib = _load()
    raw = np.ascontiguousarray(raw)
    want = np.uint16 if dtype == "bf16" else np.float32
    if raw.dtype != want:
        raise TypeError("raw must be %s for %s" % (np.dtype(want).name, dtype))
    batch, row_stride = raw.shape
    lens = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
    if lens.shape != (batch,):
        raise ValueError("one length per row")
    idx = np.zeros((batch, k), dtype=np.int32)
    val = np.zeros((batch, k), dtype=want) if return_value else None
    st = lib.oracle_topk_lengths(raw.ctypes.data, _DT[dtype], batch, n, row_stride, k, lens.ctypes.data,
                                 int(sorted_index), int(bool(return_value)), idx.ctypes.data,
                                 val.ctypes.data if val is not None else None, int(nthreads))
    return st, idx, val


def sample(raw: np.ndarray, dtype: str, n: int, k: int, temperature, top_p, uniform
           ) -> Tuple[int, np.ndarray]:
    """One token per row drawn from the row's top-k (see oracle_sample in
    oracle.c): temperature softmax over the candidates, top-p nucleus,
    inverse CDF at the caller's uniform u.  Returns (status, int32 [batch])."""
    lib = _load()
    raw = np.ascontiguousarray(raw)
    want = np.uint16 if dtype == "bf16" else np.float32
    if raw.dtype != want:
        raise TypeError("raw must be %s for %s" % (np.dtype(want).name, dtype))
    batch, row_stride = raw.shape
    f = [np.ascontiguousarray(np.broadcast_to(np.asarray(a, dtype=np.float32), (batch,)))
         for a in (temperature, top_p, uniform)]
    out = np.zeros(batch, dtype=np.int32)
    st = lib.oracle_sample(raw.ctypes.data, _DT[dtype], batch, n, row_stride, k, f[0].ctypes.data,
                           f[1].ctypes.data, f[2].ctypes.data, out.ctypes.data)
    return st, out
