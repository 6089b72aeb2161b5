"""GPU: per-row valid lengths (ds_topk_lengths) against the oracle, with the
columns past each row's length holding NaN (they must not be read), and
against ds_topk on the same rows with -inf tails (the C4 decode workload)."""

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


def _run(pkg, raw, dtype, n, k, lens, order, retval=True):
    import torch

    x = to_device(raw, dtype)
    lt = torch.tensor(np.asarray(lens, dtype=np.int32), device="cuda:0")
    val, idx = pkg.topk(x, k, sorted_index=order == 1, sorted_value=order == 2, return_value=retval, n=n,
                        lengths=lt)
    return idx.cpu().numpy(), (to_host_bits(val, dtype) if val is not None else None)


def _nan_tails(raw, dtype, lens):
    t = raw.copy()
    nan = np.uint16(0x7FC1) if dtype == "bf16" else np.float32(np.nan)
    for r, L in enumerate(lens):
        t[r, max(0, min(int(L), t.shape[1])):] = nan
    return t


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("segs", [0, 1, 4])
def test_lengths_edges(pkg, oracle_mod, dtype, segs):
    # lengths 0, 1, below k, equal to k, inside, n, above n, negative (clamped)
    n, k = 9000, 300
    lens = [0, 1, 17, 299, 300, 4321, n, n + 77, -5]
    raw = _nan_tails(make_edge_rows(dtype, len(lens), n, seed=11, levels=8, specials=0.02), dtype, lens)
    pkg.ds_topk_set_overrides(segs, 0)
    try:
        for order in (0, 1, 2):
            log("lengths edges %s segs=%d order=%d" % (dtype, segs, order))
            st, oidx, oval = oracle_mod.topk_lengths(raw, dtype, n, k, lens, order, True, nthreads=0)
            assert st == 0
            gidx, gval = _run(pkg, raw, dtype, n, k, lens, order)
            # (values: compare with the oracle's, which are -inf past the length)
            if order:
                assert np.array_equal(gidx, oidx)
            else:
                assert np.array_equal(np.sort(gidx, axis=1), np.sort(oidx, axis=1))
            o = np.argsort(gidx, axis=1, kind="stable")
            p = np.argsort(oidx, axis=1, kind="stable")
            gv = np.take_along_axis(gval, o, axis=1).view(np.uint16 if dtype == "bf16" else np.uint32)
            ov = np.take_along_axis(oval, p, axis=1).view(np.uint16 if dtype == "bf16" else np.uint32)
            assert np.array_equal(gv, ov)
    finally:
        pkg.ds_topk_set_overrides(0, 0)


@pytest.mark.parametrize("order", [0, 1, 2])
def test_lengths_equal_neg_inf_tails_on_decode_workload(pkg, oracle_mod, order):
    # The C4 rows are valid prefixes followed by -inf: ds_topk_lengths on the
    # prefix lengths (tails overwritten with NaN) gives ds_topk's answer on the
    # -inf rows and the oracle's.
    w = make_workload("C4", batch=16)
    lens = w.meta["lengths"]
    log("lengths vs -inf tails C4 batch=16 order=%d" % order)
    raw_nan = _nan_tails(w.raw, w.dtype, lens)
    gidx, gval = _run(pkg, raw_nan, w.dtype, w.n, w.k, lens, order)
    import torch

    x = to_device(w.raw, w.dtype)
    val, idx = pkg.topk(x, w.k, sorted_index=order == 1, sorted_value=order == 2, return_value=True, n=w.n)
    ridx, rval = idx.cpu().numpy(), to_host_bits(val, w.dtype)
    st, oidx, oval = oracle_mod.topk(w.raw, w.dtype, w.n, w.k, order, True, nthreads=0)
    assert st == 0
    assert_parity(w.raw, w.dtype, w.n, w.k, order, gidx, gval, oidx, oval)
    if order:
        assert np.array_equal(gidx, ridx) and np.array_equal(gval, rval)
    else:
        assert np.array_equal(np.sort(gidx, axis=1), np.sort(ridx, axis=1))


@pytest.mark.parametrize("cfg", ["C2", "C3"])
def test_lengths_full_rows_match_plain_call(pkg, cfg):
    # lengths = n everywhere: the plain call's answer
    w = make_workload(cfg, batch=4)
    log("lengths = n %s" % cfg)
    a_idx, a_val = _run(pkg, w.raw, w.dtype, w.n, w.k, [w.n] * w.batch, 1)
    x = to_device(w.raw, w.dtype)
    val, idx = pkg.topk(x, w.k, sorted_index=True, return_value=True, n=w.n)
    assert np.array_equal(a_idx, idx.cpu().numpy())
    assert np.array_equal(a_val, to_host_bits(val, w.dtype))
