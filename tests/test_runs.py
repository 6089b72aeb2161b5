"""GPU: rows holding long runs of one value, the inputs for which the seed
counts a wave's part of a tile at once: runs of +inf, -inf, a finite value
and NaN, aligned and not aligned with tiles (4096 bf16 or 2048 fp32
elements) and segments, under several forced segment counts.  Runs of
numbers are compared with the oracle element by element; a NaN run
anywhere must be reported."""

import numpy as np
import pytest

from gpu_util import assert_parity, gpu_topk, log, to_device

pytestmark = pytest.mark.gpu

DTYPES = ["bf16", "f32"]
N = 40000
# (start, length) of the run in each row
RUNS = [(0, 4096), (4096, 8192), (100, 20000), (N - 4096, 4096), (N // 2 - 3, 7), (0, N)]


@pytest.fixture(scope="module")
def pkg():
    import sampling_topk_selection_amd as p

    p.load_library()
    yield p
    p.ds_topk_set_overrides(0, 0)


def _bits(dtype, v):
    v = np.asarray(v, dtype=np.float32)
    if dtype == "f32":
        return v
    u = v.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)  # round to nearest even


def _rows(dtype, value, seed):
    rng = np.random.default_rng(seed)
    rows = []
    for start, length in RUNS:
        r = rng.standard_normal(N).astype(np.float32)
        r[start:start + length] = value
        rows.append(r)
    return np.stack([_bits(dtype, r) for r in rows])


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("value", [np.inf, -np.inf, 2.5])
def test_runs_of_one_value(pkg, oracle_mod, dtype, value):
    raw = _rows(dtype, value, seed=int(abs(value) * 10) if np.isfinite(value) else 7 + (value > 0))
    for k in (1, 512, 1025, 4096):
        st, oidx, oval = oracle_mod.topk(raw, dtype, N, k, 1, True, nthreads=0)
        assert st == 0
        for segs in (0, 1, 2, 3):
            log("runs %s value=%s k=%d segs=%d" % (dtype, value, k, segs))
            pkg.ds_topk_set_overrides(segs, 0)
            try:
                gidx, gval = gpu_topk(raw, dtype, N, k, 1, True)
            finally:
                pkg.ds_topk_set_overrides(0, 0)
            assert_parity(raw, dtype, N, k, 1, gidx, gval, oidx, oval, invariant_rows=range(raw.shape[0]))


@pytest.mark.parametrize("dtype", DTYPES)
def test_nan_runs_are_reported(pkg, dtype):
    for nan_bits in (0x7FC00000, 0xFFC00000):  # quiet NaN of either sign
        raw = _rows(dtype, np.uint32(nan_bits).view(np.float32), seed=11)
        for r in range(raw.shape[0]):
            one = raw[r:r + 1].copy()
            for k in (64, 1025):
                for segs in (0, 1, 3):
                    log("nan run %s bits=%x row=%d k=%d segs=%d" % (dtype, nan_bits, r, k, segs))
                    pkg.ds_topk_set_overrides(segs, 0)
                    try:
                        with pytest.raises(FloatingPointError):
                            pkg.topk(to_device(one, dtype), k, n=N)
                    finally:
                        pkg.ds_topk_set_overrides(0, 0)
