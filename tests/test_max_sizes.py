"""GPU: the largest sizes the boundary accepts -- a row of almost 2^31 bf16
columns (the int32 index limit) and a batch past one launch's grid.  The
oracle would take minutes here, so the answer is planted: k entries of 4.0
in rows of uniform values below 0.5, at known distinct columns; the top-k
set is exactly those columns (equal values, so ties are all inside the set),
and each value must be the bit copy of 4.0."""

import pytest

from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkg():
    import sampling_topk_selection_amd as p

    p.load_library()
    yield p
    p.ds_topk_set_overrides(0, 0)


def _planted(batch, n, k, a, b):
    import torch

    g = torch.Generator(device="cuda").manual_seed(batch * 7 + n)
    x = torch.rand((batch, n), generator=g, device="cuda", dtype=torch.bfloat16).mul_(0.5)
    rows = torch.arange(batch, device="cuda", dtype=torch.int64)[:, None]
    cols = (torch.arange(k, device="cuda", dtype=torch.int64)[None, :] * a + rows * b) % n
    x.scatter_(1, cols, 4.0)
    return x, cols


def _check(pkg, x, cols, k):
    import torch

    val, idx = pkg.topk(x, k, sorted_index=True, return_value=True)
    want = torch.sort(cols, dim=1).values.to(torch.int32)
    assert torch.equal(idx, want)
    four = torch.full_like(val, 4.0)
    assert torch.equal(val.view(torch.int16), four.view(torch.int16))


def test_longest_row(pkg):
    # n = 2^31 - 8 bf16 columns (4 GiB): indices near the int32 limit, and
    # a single forced segment that must still be split per buffer resource
    import torch

    n, k = (1 << 31) - 8, 4096
    x, cols = _planted(1, n, k, a=524287, b=0)  # 524287 = 2^19 - 1 is coprime to n
    assert int(cols.max()) > (1 << 31) - (1 << 20)  # columns near the int32 limit are selected
    for segs in (0, 1):
        log("longest row n=%d k=%d segs=%d" % (n, k, segs))
        pkg.ds_topk_set_overrides(segs, 0, 0)
        try:
            _check(pkg, x, cols, k)
        finally:
            pkg.ds_topk_set_overrides(0, 0, 0)
    del x
    torch.cuda.empty_cache()


def test_batch_past_one_launch(pkg):
    # more rows than one launch's grid holds: the call splits the batch
    import torch

    batch, n, k = (1 << 22) + 5, 2056, 8
    st, plan = pkg.ds_topk_plan_for(0, batch, n, n, k)
    assert st == 0 and plan.grid < batch, "the batch must need more than one launch"
    x, cols = _planted(batch, n, k, a=97, b=131)
    log("batch past one launch: %d rows x %d, k=%d, rows per launch %d" % (batch, n, k, plan.grid))
    _check(pkg, x, cols, k)
    del x
    torch.cuda.empty_cache()
