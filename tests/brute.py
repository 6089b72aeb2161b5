"""Brute-force rank counting, written independently of the oracle.

rank(i) = number of positions j that precede i, where j precedes i iff
v_j > v_i, or both are zeros and v_j is +0 while v_i is -0, or v_j and v_i
are the same value and j < i.  The top-k set is {i : rank(i) < k}.

Two forms: a pure-Python O(n^2) loop over struct-decoded values for tiny
rows, and a numpy O(n^2) broadcast for rows up to a few thousand.
"""

from __future__ import annotations

import math
import struct

import numpy as np


def decode(bits_row, dtype: str):
    """Python floats from raw bits (bf16 = high half of binary32)."""
    out = []
    for b in bits_row:
        if dtype == "bf16":
            u = (int(b) & 0xFFFF) << 16
        else:
            u = int(np.float32(b).view(np.uint32))
        out.append(struct.unpack("<f", struct.pack("<I", u))[0])
    return out


def precedes(vj: float, j: int, vi: float, i: int) -> bool:
    if vj > vi:
        return True
    if vj < vi:
        return False
    if vj == 0.0:
        sj, si = math.copysign(1.0, vj), math.copysign(1.0, vi)
        if sj != si:
            return sj > si
    return j < i


def topk_set_loop(bits_row, dtype: str, k: int):
    vals = decode(bits_row, dtype)
    n = len(vals)
    ranks = [sum(1 for j in range(n) if j != i and precedes(vals[j], j, vals[i], i))
             for i in range(n)]
    return sorted(i for i in range(n) if ranks[i] < k)


def _as_f64(bits_row: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (bits_row.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(bits_row, dtype=np.float32).astype(np.float64)


def topk_set_numpy(bits_row: np.ndarray, dtype: str, k: int) -> np.ndarray:
    v = _as_f64(np.asarray(bits_row), dtype)
    n = v.shape[0]
    pos = ~np.signbit(v)
    idx = np.arange(n)
    # P[j, i] = j precedes i
    gt = v[:, None] > v[None, :]
    eq = v[:, None] == v[None, :]
    zero_split = eq & (v[:, None] == 0.0) & (pos[:, None] != pos[None, :])
    P = gt | (zero_split & pos[:, None]) | (eq & ~zero_split & (idx[:, None] < idx[None, :]))
    rank = P.sum(axis=0)
    return np.nonzero(rank < k)[0]
