"""Complete O(n) check of a top-k answer, independent of any sort.

A set S of column indices is THE top-k of a row (under "larger value first,
+0 before -0, lower index first among equal values") if and only if

  * |S| = k, its indices are distinct and lie in [0, n), and
  * the least element of S precedes the greatest element outside S.

So checking this pins the selected set at any size without trusting the
oracle.  Values and the sorted order are checked bit-for-bit separately.
"""

from __future__ import annotations

import numpy as np

from brute import _as_f64, precedes


def _least(v: np.ndarray, idx: np.ndarray):
    """(value, index) of the element that every other element precedes."""
    cand = v == v.min()
    if v.min() == 0.0 and np.any(cand & np.signbit(v)):
        cand &= np.signbit(v)  # -0 comes after +0
    p = np.nonzero(cand)[0][-1]  # among identical values the highest index is last
    return float(v[p]), int(idx[p])


def _greatest(v: np.ndarray, idx: np.ndarray):
    """(value, index) of the element that precedes every other element."""
    cand = v == v.max()
    if v.max() == 0.0 and np.any(cand & ~np.signbit(v)):
        cand &= ~np.signbit(v)  # +0 comes before -0
    p = np.nonzero(cand)[0][0]  # among identical values the lowest index is first
    return float(v[p]), int(idx[p])


def check_topk_row(bits_row: np.ndarray, dtype: str, n: int, k: int, sel: np.ndarray,
                   sorted_index: bool = False) -> None:
    sel = np.asarray(sel, dtype=np.int64)
    assert sel.shape == (k,), "expected %d indices, got %s" % (k, sel.shape)
    assert np.all((sel >= 0) & (sel < n)), "index out of range"
    assert np.unique(sel).shape[0] == k, "duplicate indices"
    if sorted_index:
        assert np.all(np.diff(sel) > 0), "indices not strictly ascending"
    if k == n:
        return
    v = _as_f64(np.asarray(bits_row[:n]), dtype)
    assert not np.any(np.isnan(v)), "row holds NaN"
    idx = np.arange(n)
    in_s = np.zeros(n, dtype=bool)
    in_s[sel] = True
    lv, li = _least(v[in_s], idx[in_s])
    gv, gi = _greatest(v[~in_s], idx[~in_s])
    assert precedes(lv, li, gv, gi), (
        "selected element (%r @ %d) does not precede unselected (%r @ %d)" % (lv, li, gv, gi))


def check_values_row(bits_row: np.ndarray, sel: np.ndarray, vals: np.ndarray) -> None:
    """Returned values must be bit copies of the inputs at the indices."""
    a = np.asarray(bits_row)[np.asarray(sel, dtype=np.int64)]
    b = np.asarray(vals)
    assert a.dtype == b.dtype
    av = a.view(np.uint16 if a.dtype == np.uint16 else np.uint32)
    bv = b.view(np.uint16 if b.dtype == np.uint16 else np.uint32)
    assert np.array_equal(av, bv), "values are not bit copies of the selected inputs"
