"""Python binding of libds_topk.so (row-wise small-k top-k on MI355X).

Two layers, both argument marshalling only -- every step of the selection
runs in the library's HIP kernels:

* the C ABI under the same names (``ds_topk``, ``ds_topk_async``,
  ``ds_topk_status_string``, ``ds_topk_plan_for``, ...) taking raw device
  pointers and a stream handle;
* ``topk(x, k, sorted_index=False, return_value=True)`` for torch tensors,
  returning ``(values or None, indices)`` like the pages' usage example
  (CSDN page "DeepSeek 一次开源三个仓库", section 三).

torch supplies device memory and streams only.  It is imported before the
library is loaded so that both bind to the same HIP runtime.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch  # noqa: F401  (loads the HIP runtime the library binds to)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libds_topk.so")

DS_DTYPE_BF16 = 0
DS_DTYPE_F32 = 1

DS_OK = 0
DS_ERR_INVALID_ARGUMENT = 1
DS_ERR_UNSUPPORTED = 2
DS_ERR_MISALIGNED = 3
DS_ERR_NAN = 4
DS_ERR_HIP = 5
DS_ORDER_NONE = 0
DS_ORDER_INDEX = 1
DS_ORDER_VALUE = 2

MAX_K = 4096
DS_TOPK_NOALLOC_SCRATCH_BYTES = 16 << 20  # the no-alloc entry point's static device array

EXPORTS = ("ds_topk", "ds_topk_async", "ds_topk_async_noalloc", "ds_topk_lengths", "ds_topk_ex", "ds_topk_sample",
           "ds_topk_status_string", "ds_topk_last_error", "ds_topk_plan_for", "ds_topk_set_overrides",
           "ds_topk_release_stream", "ds_topk_version")


class TopkError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__("%s (%s)" % (ds_topk_status_string(status), detail))
        self.status = status


class ds_topk_plan(ctypes.Structure):
    _fields_ = [("segments", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("tiles_per_chunk", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("segment_vectors", ctypes.c_int32), ("tiles_per_segment", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64), ("publish_capacity", ctypes.c_int32)]


class ds_topk_options(ctypes.Structure):
    _fields_ = [("index_bytes", ctypes.c_int32), ("lengths", ctypes.c_void_p), ("status_dev", ctypes.c_void_p)]


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the in-tree libds_topk.so.  Raises if it has not been built --
    there is no fallback implementation."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError("libds_topk.so not built (%s); run python -m sampling_topk_selection_amd.build" % p)
    lib = ctypes.CDLL(p)
    i64, i32, vp, ci = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int
    lib.ds_topk.restype = ci
    lib.ds_topk.argtypes = [vp, ci, i64, i64, i64, i32, ci, ci, vp, vp, vp]
    lib.ds_topk_async.restype = ci
    lib.ds_topk_async.argtypes = [vp, ci, i64, i64, i64, i32, ci, ci, vp, vp, vp, vp]
    lib.ds_topk_async_noalloc.restype = ci
    lib.ds_topk_async_noalloc.argtypes = [vp, ci, i64, i64, i64, i32, ci, ci, vp, vp, vp, vp]
    lib.ds_topk_lengths.restype = ci
    lib.ds_topk_lengths.argtypes = [vp, ci, i64, i64, i64, i32, vp, ci, ci, vp, vp, vp]
    lib.ds_topk_sample.restype = ci
    lib.ds_topk_sample.argtypes = [vp, ci, i64, i64, i64, i32, vp, vp, vp, vp, vp]
    lib.ds_topk_ex.restype = ci
    lib.ds_topk_ex.argtypes = [vp, ci, i64, i64, i64, i32, ci, ci, vp, vp, ctypes.POINTER(ds_topk_options), vp]
    lib.ds_topk_status_string.restype = ctypes.c_char_p
    lib.ds_topk_status_string.argtypes = [ci]
    lib.ds_topk_last_error.restype = ctypes.c_char_p
    lib.ds_topk_last_error.argtypes = []
    lib.ds_topk_plan_for.restype = ci
    lib.ds_topk_plan_for.argtypes = [ci, i64, i64, i64, i32, ci, ci, ctypes.POINTER(ds_topk_plan)]
    lib.ds_topk_set_overrides.restype = None
    lib.ds_topk_set_overrides.argtypes = [i32, ctypes.c_uint32, i32]
    lib.ds_topk_release_stream.restype = ci
    lib.ds_topk_release_stream.argtypes = [vp]
    lib.ds_topk_version.restype = ci
    lib.ds_topk_version.argtypes = []
    if path is None:
        _lib = lib
    return lib


# ------------------------------------------------------------------ C ABI, same names
def ds_topk(in_ptr: int, dtype: int, batch: int, n: int, row_stride: int, k: int, sorted_index: int,
            return_value: int, out_idx_ptr: int, out_val_ptr: Optional[int], stream: Optional[int]) -> int:
    return load_library().ds_topk(in_ptr, dtype, batch, n, row_stride, k, sorted_index, return_value,
                                  out_idx_ptr, out_val_ptr, stream)


def ds_topk_lengths(in_ptr: int, dtype: int, batch: int, n: int, row_stride: int, k: int,
                    lengths_ptr: Optional[int], sorted_index: int, return_value: int, out_idx_ptr: int,
                    out_val_ptr: Optional[int], stream: Optional[int]) -> int:
    return load_library().ds_topk_lengths(in_ptr, dtype, batch, n, row_stride, k, lengths_ptr, sorted_index,
                                          return_value, out_idx_ptr, out_val_ptr, stream)


def ds_topk_ex(in_ptr: int, dtype: int, batch: int, n: int, row_stride: int, k: int, sorted_index: int,
               return_value: int, out_idx_ptr: int, out_val_ptr: Optional[int], index_bytes: int = 4,
               lengths_ptr: Optional[int] = None, status_dev_ptr: Optional[int] = None,
               stream: Optional[int] = None) -> int:
    opt = ds_topk_options(index_bytes, lengths_ptr, status_dev_ptr)
    return load_library().ds_topk_ex(in_ptr, dtype, batch, n, row_stride, k, sorted_index, return_value,
                                     out_idx_ptr, out_val_ptr, ctypes.byref(opt), stream)


def ds_topk_sample(in_ptr: int, dtype: int, batch: int, n: int, row_stride: int, k: int, temperature_ptr: int,
                   top_p_ptr: int, uniform_ptr: int, out_token_ptr: int, stream: Optional[int]) -> int:
    return load_library().ds_topk_sample(in_ptr, dtype, batch, n, row_stride, k, temperature_ptr, top_p_ptr,
                                         uniform_ptr, out_token_ptr, stream)


def ds_topk_async(in_ptr: int, dtype: int, batch: int, n: int, row_stride: int, k: int, sorted_index: int,
                  return_value: int, out_idx_ptr: int, out_val_ptr: Optional[int], status_dev_ptr: int,
                  stream: Optional[int]) -> int:
    return load_library().ds_topk_async(in_ptr, dtype, batch, n, row_stride, k, sorted_index, return_value,
                                        out_idx_ptr, out_val_ptr, status_dev_ptr, stream)


def ds_topk_async_noalloc(in_ptr: int, dtype: int, batch: int, n: int, row_stride: int, k: int, sorted_index: int,
                          return_value: int, out_idx_ptr: int, out_val_ptr: Optional[int], status_dev_ptr: int,
                          stream: Optional[int]) -> int:
    return load_library().ds_topk_async_noalloc(in_ptr, dtype, batch, n, row_stride, k, sorted_index, return_value,
                                                out_idx_ptr, out_val_ptr, status_dev_ptr, stream)


def ds_topk_status_string(status: int) -> str:
    return load_library().ds_topk_status_string(status).decode()


def ds_topk_last_error() -> str:
    return load_library().ds_topk_last_error().decode()


def ds_topk_plan_for(dtype: int, batch: int, n: int, row_stride: int, k: int, sorted_index: int = 0,
                     return_value: int = 1) -> Tuple[int, ds_topk_plan]:
    plan = ds_topk_plan()
    st = load_library().ds_topk_plan_for(dtype, batch, n, row_stride, k, sorted_index, return_value,
                                         ctypes.byref(plan))
    return st, plan


DS_TOPK_FORCE_BITONIC = 1


def ds_topk_set_overrides(segments: int = 0, tile_seed: int = 0, flags: int = 0) -> None:
    """Overrides for the calling thread's calls (tests and measurements)."""
    load_library().ds_topk_set_overrides(segments, tile_seed, flags)


def ds_topk_release_stream(stream: Optional[int]) -> int:
    return load_library().ds_topk_release_stream(stream)


def ds_topk_version() -> int:
    return load_library().ds_topk_version()


# ------------------------------------------------------------------ torch convenience
_TORCH_DT = {torch.bfloat16: DS_DTYPE_BF16, torch.float32: DS_DTYPE_F32}


def _check(st: int) -> None:
    if st == DS_OK:
        return
    detail = ds_topk_last_error()
    if st in (DS_ERR_INVALID_ARGUMENT, DS_ERR_UNSUPPORTED, DS_ERR_MISALIGNED):
        raise ValueError("%s (%s)" % (ds_topk_status_string(st), detail))
    if st == DS_ERR_NAN:
        raise FloatingPointError("%s (%s)" % (ds_topk_status_string(st), detail))
    raise TopkError(st, detail)


def _marshal(x: torch.Tensor, k: int, n: Optional[int]):
    if x.dtype not in _TORCH_DT:
        raise ValueError("dtype %s unsupported: bfloat16 or float32 only" % x.dtype)
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    if x.dim() == 1:
        x = x.unsqueeze(0)
    if x.dim() != 2 or (x.shape[1] > 1 and x.stride(1) != 1):
        raise ValueError("x must be [batch, n] with unit stride along n")
    batch = x.shape[0]
    n = x.shape[1] if n is None else n
    row_stride = x.stride(0) if batch > 1 else max(x.stride(0), x.shape[1])
    return x, _TORCH_DT[x.dtype], batch, n, row_stride


def _order(sorted_index: bool, sorted_value: bool) -> int:
    if sorted_index and sorted_value:
        raise ValueError("sorted_index and sorted_value are exclusive")
    return DS_ORDER_VALUE if sorted_value else DS_ORDER_INDEX if sorted_index else DS_ORDER_NONE


_INDEX_BYTES = {torch.int32: 4, torch.int64: 8}


def _lengths_ptr(lengths: Optional[torch.Tensor], batch: int) -> Optional[int]:
    if lengths is None:
        return None
    if lengths.dtype != torch.int32 or not lengths.is_cuda or lengths.numel() != batch or \
            not lengths.is_contiguous():
        raise ValueError("lengths must be a contiguous int32 device tensor with one entry per row")
    return lengths.data_ptr()


def topk(x: torch.Tensor, k: int, *, sorted_index: bool = False, return_value: bool = True,
         n: Optional[int] = None, sorted_value: bool = False, lengths: Optional[torch.Tensor] = None,
         indices_type: torch.dtype = torch.int32) -> Tuple[Optional[torch.Tensor], torch.Tensor]:
    """Top-k of each row of ``x`` ([batch, n], bf16 or fp32, on the device).

    Returns ``(values, indices)``; values is None when ``return_value`` is
    False.  Indices are ``indices_type``.  ``sorted_index`` writes each row's indices in
    ascending order, ``sorted_value`` largest value first (ties by lower
    index); neither leaves the order free.  ``n`` restricts the selection to
    the first n columns (the rest of each row is padding).  ``lengths`` (an
    int32 device tensor, one per row) gives each row's own valid length: the
    columns past it act as -inf and are not read.  ``indices_type`` is
    torch.int32 or torch.int64.  Blocks until done.
    """
    order = _order(sorted_index, sorted_value)
    if indices_type not in _INDEX_BYTES:
        raise ValueError("indices_type must be torch.int32 or torch.int64")
    x, dt, batch, n, row_stride = _marshal(x, k, n)
    idx = torch.empty((batch, k), dtype=indices_type, device=x.device)
    val = torch.empty((batch, k), dtype=x.dtype, device=x.device) if return_value else None
    stream = torch.cuda.current_stream(x.device).cuda_stream
    if lengths is not None or indices_type != torch.int32:
        st = ds_topk_ex(x.data_ptr(), dt, batch, n, row_stride, k, order, int(bool(return_value)), idx.data_ptr(),
                        val.data_ptr() if val is not None else None, _INDEX_BYTES[indices_type],
                        _lengths_ptr(lengths, batch), None, stream)
    else:
        st = ds_topk(x.data_ptr(), dt, batch, n, row_stride, k, order, int(bool(return_value)),
                     idx.data_ptr(), val.data_ptr() if val is not None else None, stream)
    _check(st)
    return val, idx


def _check_out(x: torch.Tensor, batch: int, k: int, val: Optional[torch.Tensor], idx: torch.Tensor,
               return_value: bool) -> None:
    """Preallocated outputs must be what the kernels write: contiguous
    (batch, k) tensors on x's device, indices int32/int64, values in x's
    dtype (when values are returned)."""
    def ok(t):
        return (isinstance(t, torch.Tensor) and tuple(t.shape) == (batch, k) and t.is_contiguous()
                and t.device == x.device)
    if not ok(idx) or idx.dtype not in _INDEX_BYTES:
        raise ValueError("out indices must be a contiguous (%d, %d) int32 or int64 tensor on %s" % (batch, k, x.device))
    if return_value and (not ok(val) or val.dtype != x.dtype):
        raise ValueError("out values must be a contiguous (%d, %d) %s tensor on %s" % (batch, k, x.dtype, x.device))


def topk_async(x: torch.Tensor, k: int, status: torch.Tensor, *, sorted_index: bool = False,
               return_value: bool = True, n: Optional[int] = None,
               out: Optional[Tuple[Optional[torch.Tensor], torch.Tensor]] = None, sorted_value: bool = False,
               lengths: Optional[torch.Tensor] = None, indices_type: torch.dtype = torch.int32
               ) -> Tuple[Optional[torch.Tensor], torch.Tensor]:
    """Enqueue the selection on the current stream without waiting.

    ``status`` is a zero-initialised int32 device tensor (one element); the
    kernels store DS_ERR_NAN there if a row holds NaN.  ``out`` may supply
    preallocated (values, indices).  Other arguments as for topk()."""
    order = _order(sorted_index, sorted_value)
    x, dt, batch, n, row_stride = _marshal(x, k, n)
    if out is not None:
        val, idx = out
        _check_out(x, batch, k, val, idx, return_value)
        indices_type = idx.dtype
    else:
        idx = torch.empty((batch, k), dtype=indices_type, device=x.device)
        val = torch.empty((batch, k), dtype=x.dtype, device=x.device) if return_value else None
    if indices_type not in _INDEX_BYTES:
        raise ValueError("indices must be torch.int32 or torch.int64")
    if status.dtype != torch.int32 or not status.is_cuda:
        raise ValueError("status must be an int32 device tensor")
    stream = torch.cuda.current_stream(x.device).cuda_stream
    if lengths is not None or indices_type != torch.int32:
        st = ds_topk_ex(x.data_ptr(), dt, batch, n, row_stride, k, order, int(bool(return_value)), idx.data_ptr(),
                        val.data_ptr() if val is not None else None, _INDEX_BYTES[indices_type],
                        _lengths_ptr(lengths, batch), status.data_ptr(), stream)
    else:
        st = ds_topk_async(x.data_ptr(), dt, batch, n, row_stride, k, order,
                           int(bool(return_value)), idx.data_ptr(), val.data_ptr() if val is not None else None,
                           status.data_ptr(), stream)
    _check(st)
    return val, idx


def sample(x: torch.Tensor, k: int, temperature, top_p, uniform, *, n: Optional[int] = None) -> torch.Tensor:
    """One token per row of ``x`` drawn from its top-k (see ds_topk_sample in
    include/ds_topk.h): temperature softmax over the k candidates, top-p
    nucleus, inverse CDF at ``uniform``.  ``temperature``, ``top_p`` and
    ``uniform`` are floats or float32 device tensors with one entry per row.
    Returns int32 [batch] column indices.  Blocks until done."""
    x, dt, batch, n, row_stride = _marshal(x, k, n)

    def per_row(a, name):
        if isinstance(a, torch.Tensor):
            if a.dtype != torch.float32 or not a.is_cuda or a.numel() != batch or not a.is_contiguous():
                raise ValueError("%s must be a contiguous float32 device tensor with one entry per row" % name)
            return a
        return torch.full((batch,), float(a), dtype=torch.float32, device=x.device)

    t, p, u = per_row(temperature, "temperature"), per_row(top_p, "top_p"), per_row(uniform, "uniform")
    out = torch.empty(batch, dtype=torch.int32, device=x.device)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    _check(ds_topk_sample(x.data_ptr(), dt, batch, n, row_stride, k, t.data_ptr(), p.data_ptr(), u.data_ptr(),
                          out.data_ptr(), stream))
    return out
