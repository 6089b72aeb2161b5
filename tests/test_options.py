"""GPU: ds_topk_ex options -- int64 indices, per-row lengths, enqueue-only
with a status word -- against the oracle and against the plain entry point."""

import numpy as np
import pytest

from gpu_util import assert_parity, log, to_device, to_host_bits
from workloads import make_edge_rows, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkg():
    import sampling_topk_selection_amd as p

    p.load_library()
    yield p
    p.ds_topk_set_overrides(0, 0)


@pytest.mark.parametrize("cfg", ["C1", "C3", "C5"])
@pytest.mark.parametrize("order", [0, 1, 2])
def test_int64_indices(pkg, oracle_mod, cfg, order):
    import torch

    w = make_workload(cfg, batch=4)
    log("int64 indices %s order=%d" % (cfg, order))
    x = to_device(w.raw, w.dtype)
    val, idx = pkg.topk(x, w.k, sorted_index=order == 1, sorted_value=order == 2, n=w.n, indices_type=torch.int64)
    assert idx.dtype == torch.int64
    gidx = idx.cpu().numpy()
    assert gidx.min() >= 0 and gidx.max() < w.n
    st, oidx, oval = oracle_mod.topk(w.raw, w.dtype, w.n, w.k, order, True, nthreads=0)
    assert st == 0
    assert_parity(w.raw, w.dtype, w.n, w.k, order, gidx.astype(np.int32), to_host_bits(val, w.dtype), oidx, oval)


def test_int64_with_lengths_and_status_word(pkg, oracle_mod):
    import torch

    n, k = 5000, 700
    lens = [0, 3, 699, 700, 2500, n]
    raw = make_edge_rows("f32", len(lens), n, seed=21, levels=16, specials=0.03)
    raw[2, 699:] = np.nan  # past its length: never looked at
    x = to_device(raw, "f32")
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    for order in (0, 1, 2):
        log("int64 + lengths + status order=%d" % order)
        val, idx = pkg.topk_async(x, k, status, sorted_index=order == 1, sorted_value=order == 2, n=n, lengths=lt,
                                  indices_type=torch.int64)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        st, oidx, oval = oracle_mod.topk_lengths(raw, "f32", n, k, lens, order, True, nthreads=0)
        assert st == 0
        gidx = idx.cpu().numpy()
        gval = to_host_bits(val, "f32")
        if order:
            assert np.array_equal(gidx, oidx)
            assert np.array_equal(gval.view(np.uint32), oval.view(np.uint32))
        else:
            assert np.array_equal(np.sort(gidx, axis=1), np.sort(oidx, axis=1))
    # a NaN inside a length is reported through the status word
    raw[4, 10] = np.nan
    x = to_device(raw, "f32")
    pkg.topk_async(x, k, status, n=n, lengths=lt, indices_type=torch.int64)
    torch.cuda.synchronize()
    assert int(status.item()) == pkg.DS_ERR_NAN
