"""ds_topk_async_noalloc (split-row state in the library's static device
array, no allocation) against ds_topk_async (the per-stream workspace) on the
same inputs, through the C ABI: indices equal (as sets per row where no order
is asked for), values equal bit for bit, status untouched."""

from __future__ import annotations

import numpy as np
import pytest

from gpu_util import log

pytestmark = pytest.mark.gpu


def _device_input(w):
    import torch

    raw = np.ascontiguousarray(w.raw)
    t = torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16) if w.dtype == "bf16" else torch.from_numpy(raw)
    return t.to("cuda:0")


def _call(entry, x, w, order):
    import torch

    import sampling_topk_selection_amd as pkg

    dt = pkg.DS_DTYPE_BF16 if w.dtype == "bf16" else pkg.DS_DTYPE_F32
    idx = torch.full((w.batch, w.k), -7, dtype=torch.int32, device=x.device)
    val = torch.zeros((w.batch, w.k), dtype=x.dtype, device=x.device) if w.return_value else None
    status = torch.zeros(1, dtype=torch.int32, device=x.device)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    st = entry(x.data_ptr(), dt, w.batch, w.n, w.row_stride, w.k, order, int(w.return_value), idx.data_ptr(),
               val.data_ptr() if val is not None else None, status.data_ptr(), stream)
    assert st == 0, pkg.ds_topk_last_error()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return idx, val


def _compare(a, b, order):
    import torch

    ia, va = a
    ib, vb = b
    assert ia.shape == ib.shape
    if order:
        assert torch.equal(ia, ib)
        if va is not None:
            assert torch.equal(va.view(torch.int16) if va.dtype == torch.bfloat16 else va.view(torch.int32),
                               vb.view(torch.int16) if vb.dtype == torch.bfloat16 else vb.view(torch.int32))
    else:
        sa, pa = torch.sort(ia, dim=1)
        sb, pb = torch.sort(ib, dim=1)
        assert torch.equal(sa, sb)
        if va is not None:
            bits = (lambda v: v.view(torch.int16)) if va.dtype == torch.bfloat16 else (lambda v: v.view(torch.int32))
            assert torch.equal(bits(torch.gather(va, 1, pa)), bits(torch.gather(vb, 1, pb)))


def _case(cfg, **kw):
    import sampling_topk_selection_amd as pkg
    from workloads import make_workload

    w = make_workload(cfg, **kw)
    order = int(w.sorted_index)
    log("no-alloc case %s %s %dx%d k=%d order=%d values=%d" % (cfg, w.dtype, w.batch, w.n, w.k, order,
                                                              int(w.return_value)))
    plan = pkg.ds_topk_plan()
    import ctypes

    dt = pkg.DS_DTYPE_BF16 if w.dtype == "bf16" else pkg.DS_DTYPE_F32
    assert pkg.load_library().ds_topk_plan_for(dt, w.batch, w.n, w.row_stride, w.k, order,
                                               int(w.return_value), ctypes.byref(plan)) == 0
    x = _device_input(w)
    ref = _call(pkg.ds_topk_async, x, w, order)
    got = _call(pkg.ds_topk_async_noalloc, x, w, order)
    _compare(ref, got, order)
    return plan


def test_noalloc_matches_workspace_path_two_calls():
    """Two calls in a row, the second on a smaller input with another layout
    of the hand-off state (64 rows of 4 segments, then 4 rows of 25)."""
    p1 = _case("C3")
    p2 = _case("C2")
    assert p1.segments > 1 and p2.segments > 1


def test_noalloc_batch_split_to_fit_the_scratch():
    """k = 4096 over 4 segments: 64 rows need more state than the array
    holds, so the rows run as two launches that reuse it."""
    import sampling_topk_selection_amd as pkg

    plan = _case("C5", batch=64, n=262144)
    assert plan.segments == 4
    per_row = plan.segments * (32 + 4 * 2048 + 8 * plan.publish_capacity)
    assert 64 * per_row > pkg.DS_TOPK_NOALLOC_SCRATCH_BYTES
    _case("C1")  # and a smaller call after it


def test_noalloc_rejects_a_row_beyond_the_scratch():
    import torch

    import sampling_topk_selection_amd as pkg

    n, k = 1 << 23, 4096  # 256 segments of 9216 published entries: ~21 MB for one row
    x = torch.zeros((1, n), dtype=torch.bfloat16, device="cuda:0")
    idx = torch.full((1, k), -7, dtype=torch.int32, device="cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    torch.cuda.synchronize()
    st = pkg.ds_topk_async_noalloc(x.data_ptr(), pkg.DS_DTYPE_BF16, 1, n, n, k, 0, 0, idx.data_ptr(), None,
                                   status.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == pkg.DS_ERR_UNSUPPORTED
    assert "static scratch" in pkg.ds_topk_last_error()
    torch.cuda.synchronize()
    assert bool((idx == -7).all()) and int(status.item()) == 0
