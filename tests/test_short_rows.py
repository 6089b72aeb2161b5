"""GPU: rows of at most 2048 columns take one wave each (several rows per
workgroup); parity with the oracle over lengths, k, orders, ties and
specials, per-row lengths, int64 indices and NaN reporting."""

import numpy as np
import pytest

from gpu_util import assert_parity, gpu_topk, log, to_device, to_host_bits
from workloads import make_edge_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkg():
    import sampling_topk_selection_amd as p

    p.load_library()
    p.ds_topk_set_overrides(0, 0)
    yield p


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n", [1, 63, 64, 65, 128, 255, 256, 257, 500, 2048])
@pytest.mark.parametrize("levels", [0, 5])
def test_short_rows_parity(pkg, oracle_mod, dtype, n, levels):
    raw = make_edge_rows(dtype, 9, n, seed=n * 3 + levels, levels=levels, specials=0.04)
    st, plan = pkg.ds_topk_plan_for(0 if dtype == "bf16" else 1, 9, n, raw.shape[1], 1)
    assert st == 0 and plan.segments == 0  # the one-wave-per-row kernel
    for k in sorted({1, min(n, 17), max(1, n // 2), n}):
        for order in (0, 1, 2):
            log("short rows %s n=%d k=%d levels=%d order=%d" % (dtype, n, k, levels, order))
            st, oidx, oval = oracle_mod.topk(raw, dtype, n, k, order, True, nthreads=0)
            assert st == 0
            gidx, gval = gpu_topk(raw, dtype, n, k, order, True)
            assert_parity(raw, dtype, n, k, order, gidx, gval, oidx, oval, invariant_rows=range(3))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_short_rows_lengths_int64_nan(pkg, oracle_mod, dtype):
    import torch

    n, k = 700, 40
    lens = [0, 5, 39, 40, 41, 700, 999, -3, 350]
    raw = make_edge_rows(dtype, len(lens), n, seed=4, levels=9, specials=0.05)
    nan = np.uint16(0x7FC1) if dtype == "bf16" else np.float32(np.nan)
    for r, L in enumerate(lens):
        raw[r, max(0, min(L, n)):] = nan  # past the length: never looked at
    x = to_device(raw, dtype)
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    for order in (0, 1, 2):
        log("short rows lengths int64 %s order=%d" % (dtype, order))
        val, idx = pkg.topk(x, k, sorted_index=order == 1, sorted_value=order == 2, n=n, lengths=lt,
                            indices_type=torch.int64)
        st, oidx, oval = oracle_mod.topk_lengths(raw, dtype, n, k, lens, order, True, nthreads=0)
        assert st == 0
        gidx = idx.cpu().numpy()
        gval = to_host_bits(val, dtype)
        if order:
            assert np.array_equal(gidx, oidx)
            assert np.array_equal(gval, oval)
        else:
            o, q = np.argsort(gidx, axis=1), np.argsort(oidx, axis=1)
            assert np.array_equal(np.take_along_axis(gidx, o, 1), np.take_along_axis(oidx, q, 1))
            assert np.array_equal(np.take_along_axis(gval, o, 1), np.take_along_axis(oval, q, 1))
    if raw.shape[1] > n:
        raw[6, n] = nan  # padding past n: ignored
    raw[5, 3] = nan    # inside row 5's length: reported
    with pytest.raises(FloatingPointError):
        pkg.topk(to_device(raw, dtype), k, n=n, lengths=lt)


def test_short_rows_many(pkg, oracle_mod):
    # many rows: several workgroups, a partial last one
    raw = make_edge_rows("bf16", 1027, 256, seed=12, levels=0, specials=0.0)
    st, oidx, oval = oracle_mod.topk(raw, "bf16", 256, 64, 1, True, nthreads=0)
    assert st == 0
    gidx, gval = gpu_topk(raw, "bf16", 256, 64, 1, True)
    assert_parity(raw, "bf16", 256, 64, 1, gidx, gval, oidx, oval)
