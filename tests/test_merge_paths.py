"""GPU: the merge of split rows against the oracle, at forced segment counts
on both sides of the few-segment row bin (up to 16 segments whose digit
directories are short: every wave works out the row bin from cumulative
counts) and of the row histogram (more segments, or a directory longer than
its cached head: values over a wide range of magnitudes put the row's
entries in many top-digit bins), for ties as well, in all three orders."""

import numpy as np
import pytest

from gpu_util import assert_parity, gpu_topk, log
from workloads import bf16_bits_from_f32, make_edge_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkg():
    import sampling_topk_selection_amd as p

    p.load_library()
    yield p
    p.ds_topk_set_overrides(0, 0)


def _rows(dtype, dist, batch, n, seed):
    if dist == "ties":
        return make_edge_rows(dtype, batch, n, seed=seed, levels=12)
    rng = np.random.default_rng(seed)
    if dist == "normal":
        x = rng.standard_normal((batch, n), dtype=np.float32)
    else:  # "wide": magnitudes from e^-40 to e^40, either sign
        x = (np.exp(rng.uniform(-40.0, 40.0, (batch, n))) * rng.choice([-1.0, 1.0], (batch, n))).astype(np.float32)
    return bf16_bits_from_f32(x) if dtype == "bf16" else x


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dist", ["normal", "wide", "ties"])
@pytest.mark.parametrize("segs", [2, 5, 16, 17, 31])
def test_merge_row_bin_paths(pkg, oracle_mod, dtype, dist, segs):
    n, batch = 60000, 3
    raw = _rows(dtype, dist, batch, n, seed=segs * 31 + len(dist))
    for k in (64, 700):
        want = {}
        for order in (1, 2):
            st, oi, ov = oracle_mod.topk(raw, dtype, n, k, order, True, nthreads=0)
            assert st == 0
            want[order] = (oi, ov)
        want[0] = want[2]  # any order: the index sets are compared
        for order in (0, 1, 2):
            log("merge %s %s segs=%d k=%d order=%d" % (dtype, dist, segs, k, order))
            pkg.ds_topk_set_overrides(segs, 0)
            try:
                gidx, gval = gpu_topk(raw, dtype, n, k, order, True)
            finally:
                pkg.ds_topk_set_overrides(0, 0)
            assert_parity(raw, dtype, n, k, order, gidx, gval, *want[order], invariant_rows=range(batch))
