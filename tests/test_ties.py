"""GPU against the oracle on rows made of long runs of one value, the inputs
for which the seed bound is tied (a crowded bin that holds a single value):
monotone rows of few levels, -inf tails and heads whose lengths fall on and
around tile and segment edges, a run of one value across the k-th position,
and constant rows; under several forced segment counts and tile orders, so
the end tiles are loaded from every position in the visiting order."""

import numpy as np
import pytest

from gpu_util import assert_parity, gpu_topk, log

pytestmark = pytest.mark.gpu

DTYPES = ["bf16", "f32"]


@pytest.fixture(scope="module")
def pkg():
    import sampling_topk_selection_amd as p

    p.load_library()
    yield p
    p.ds_topk_set_overrides(0, 0)


def _bits(dtype, vals):
    v = np.asarray(vals, dtype=np.float32)
    if dtype == "f32":
        return v
    u = v.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)  # round to nearest even


def _rows(dtype, n, seed):
    rng = np.random.default_rng(seed)
    levels = np.arange(-3.5, 4.0, 1.0, dtype=np.float32)  # 8 levels, exact in bf16
    rows = []
    ids = np.sort(rng.integers(0, 8, size=n))
    rows.append(levels[ids])                      # ascending levels
    rows.append(levels[ids[::-1]])                # descending levels
    for L in (0, 4096, 4097, n // 2, n - 1):      # -inf tails (L valid first)
        r = rng.standard_normal(n).astype(np.float32)
        r[L:] = -np.inf
        rows.append(r)
    r = rng.standard_normal(n).astype(np.float32)
    r[: n - 3000] = -np.inf                       # -inf head, valid end
    rows.append(r)
    r = rng.standard_normal(n).astype(np.float32)
    r[n // 3: n // 3 + 6000] = 2.5                # a run of one value across the k-th
    rows.append(r)
    rows.append(np.full(n, 1.25, dtype=np.float32))  # constant
    return np.stack([_bits(dtype, x) for x in rows])


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n", [40000, 65536])
def test_tied_seed_rows(pkg, oracle_mod, dtype, n):
    raw = _rows(dtype, n, seed=n)
    for k in (1, 512, 1500, 4096):
        st, oidx, oval = oracle_mod.topk(raw, dtype, n, k, 1, True, nthreads=0)
        assert st == 0
        for segs in (0, 1, 3, 7):
            for tile_seed in (0, 0x1234567):
                log("ties %s n=%d k=%d segs=%d tile_seed=%x" % (dtype, n, k, segs, tile_seed))
                pkg.ds_topk_set_overrides(segs, tile_seed)
                try:
                    gidx, gval = gpu_topk(raw, dtype, n, k, 1, True)
                finally:
                    pkg.ds_topk_set_overrides(0, 0)
                assert_parity(raw, dtype, n, k, 1, gidx, gval, oidx, oval, invariant_rows=range(raw.shape[0]))
