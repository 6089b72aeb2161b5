"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
library, and compare with the oracle element by element."""

from __future__ import annotations

import sys

import numpy as np

from invariants import check_topk_row, check_values_row


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(raw: np.ndarray, dtype: str):
    import torch

    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(raw))
    return t.to("cuda:0")


def to_host_bits(val, dtype: str) -> np.ndarray:
    import torch

    if dtype == "bf16":
        return val.cpu().view(torch.int16).numpy().view(np.uint16)
    return val.cpu().numpy()


def gpu_topk(raw: np.ndarray, dtype: str, n: int, k: int, sorted_index, return_value: bool):
    """sorted_index: 0/False any order, 1/True ascending index, 2 by value."""
    import sampling_topk_selection_amd as pkg

    x = to_device(raw, dtype)
    order = int(sorted_index)
    val, idx = pkg.topk(x, k, sorted_index=order == 1, sorted_value=order == 2, return_value=return_value, n=n)
    gidx = idx.cpu().numpy()
    gval = to_host_bits(val, dtype) if val is not None else None
    return gidx, gval


def assert_parity(raw: np.ndarray, dtype: str, n: int, k: int, sorted_index, gidx: np.ndarray,
                  gval, oidx: np.ndarray, oval, invariant_rows=None) -> None:
    """Indices: same set per row (same order too when an order is asked for:
    sorted_index 1 by index, 2 by value); values: bit copies of the inputs
    at the returned indices, equal to the oracle's."""
    batch = raw.shape[0]
    assert gidx.shape == (batch, k), gidx.shape
    if sorted_index:
        bad = np.nonzero(np.any(gidx != oidx, axis=1))[0]
        assert bad.size == 0, "rows %s differ from the oracle (sorted)" % bad[:8].tolist()
    else:
        g = np.sort(gidx, axis=1)
        o = np.sort(oidx, axis=1)
        bad = np.nonzero(np.any(g != o, axis=1))[0]
        assert bad.size == 0, "rows %s: index sets differ from the oracle" % bad[:8].tolist()
        assert all(np.unique(gidx[r]).size == k for r in range(batch)), "duplicate indices"
    if gval is not None:
        rows = np.arange(batch)[:, None]
        want = raw[rows, gidx.astype(np.int64)]
        wv = want.view(np.uint16 if dtype == "bf16" else np.uint32)
        gv = np.ascontiguousarray(gval).view(np.uint16 if dtype == "bf16" else np.uint32)
        assert np.array_equal(wv, gv), "values are not bit copies of the inputs"
        if sorted_index and oval is not None:
            ov = np.ascontiguousarray(oval).view(np.uint16 if dtype == "bf16" else np.uint32)
            assert np.array_equal(gv, ov)
    for r in (invariant_rows if invariant_rows is not None else []):
        check_topk_row(raw[r], dtype, n, k, gidx[r], sorted_index=int(sorted_index) == 1)
        if gval is not None:
            check_values_row(raw[r], gidx[r], gval[r])
