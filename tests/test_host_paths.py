"""GPU: the host side's refusals and stream housekeeping.

* topk_async(out=...) rejects outputs the kernels would overrun or fill with
  the wrong type, before anything is enqueued;
* a call that would have to grow a stream's workspace while the stream is
  capturing, and any synchronous call under capture, return DS_ERR_HIP and
  enqueue nothing;
* ds_topk_release_stream frees a stream's buffers, and later calls on the
  stream allocate them again and give the same answer.
"""

import pytest

from gpu_util import log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkg():
    import sampling_topk_selection_amd as p

    p.load_library()
    return p


def test_out_tensors_are_checked(pkg):
    import torch

    x = torch.randn(4, 1024, device="cuda:0").to(torch.bfloat16)
    k = 8
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    good_v = torch.empty((4, k), dtype=x.dtype, device=x.device)
    good_i = torch.empty((4, k), dtype=torch.int32, device=x.device)
    bad = [
        ("index shape", (good_v, torch.empty((4, k - 1), dtype=torch.int32, device=x.device))),
        ("index stride", (good_v, torch.empty((k, 4), dtype=torch.int32, device=x.device).t())),
        ("index dtype", (good_v, torch.empty((4, k), dtype=torch.float32, device=x.device))),
        ("index device", (good_v, torch.empty((4, k), dtype=torch.int32))),
        ("value shape", (torch.empty((3, k), dtype=x.dtype, device=x.device), good_i)),
        ("value dtype", (torch.empty((4, k), dtype=torch.float32, device=x.device), good_i)),
        ("value stride", (torch.empty((k, 4), dtype=x.dtype, device=x.device).t(), good_i)),
    ]
    marker = torch.full_like(good_i, -5)
    for name, out in bad:
        log("out check: %s" % name)
        with pytest.raises(ValueError):
            pkg.topk_async(x, k, status, out=out)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    # and the well-formed pair works
    good_i.copy_(marker)
    pkg.topk_async(x, k, status, out=(good_v, good_i))
    torch.cuda.synchronize()
    assert int((good_i >= 0).all().item())


def test_capture_refusals(pkg):
    import torch

    from workloads import make_workload

    w = make_workload("C3", batch=4)  # 4 long rows: a split plan with a workspace
    x = to_device(w.raw, w.dtype)
    st, plan = pkg.ds_topk_plan_for(pkg.DS_DTYPE_F32, w.batch, w.n, w.row_stride, w.k, 1, 1)
    assert st == 0 and plan.segments > 1 and plan.workspace_bytes > 0
    idx = torch.empty((w.batch, w.k), dtype=torch.int32, device="cuda:0")
    val = torch.empty((w.batch, w.k), dtype=torch.float32, device="cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    s = torch.cuda.Stream()  # fresh: no workspace yet
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    rcs = []
    log("capture refusals")
    with torch.cuda.graph(g, stream=s):
        idx.fill_(-3)  # (some captured work of the caller's own)
        rcs.append(pkg.ds_topk_async(x.data_ptr(), pkg.DS_DTYPE_F32, w.batch, w.n, w.row_stride, w.k, 1, 1,
                                     idx.data_ptr(), val.data_ptr(), status.data_ptr(), s.cuda_stream))
        rcs.append(pkg.ds_topk(x.data_ptr(), pkg.DS_DTYPE_F32, w.batch, w.n, w.row_stride, w.k, 1, 1,
                               idx.data_ptr(), val.data_ptr(), s.cuda_stream))
    assert rcs == [pkg.DS_ERR_HIP, pkg.DS_ERR_HIP], rcs
    g.replay()
    torch.cuda.synchronize()
    assert bool((idx == -3).all()), "a refused call enqueued work"
    assert int(status.item()) == 0
    pkg.ds_topk_release_stream(s.cuda_stream)


def test_release_stream_then_reuse(pkg):
    import torch

    from workloads import make_workload

    w = make_workload("C2")
    x = to_device(w.raw, w.dtype)
    s = torch.cuda.Stream()
    outs = []
    for rep in range(2):
        with torch.cuda.stream(s):
            v, i = pkg.topk(x, w.k, sorted_index=True, return_value=False, n=w.n)
        torch.cuda.synchronize()
        outs.append(i.cpu())
        assert pkg.ds_topk_release_stream(s.cuda_stream) == pkg.DS_OK, pkg.ds_topk_last_error()
    assert torch.equal(outs[0], outs[1])
    # releasing a stream with nothing on it is a no-op
    assert pkg.ds_topk_release_stream(s.cuda_stream) == pkg.DS_OK
