"""GPU against the oracle for the tile visiting order of the bf16 kernel for
k > 1024, which visits a segment's last and first tiles before the others:
segments of 1 to 9 tiles (whole and ragged last tiles), sorted rows both
ways, random rows, a -inf tail and a constant row, under forced segment
counts and tile orders."""

import numpy as np
import pytest

from gpu_util import assert_parity, gpu_topk, log
from workloads.gen import pad_rows

pytestmark = pytest.mark.gpu

TILE = 4096  # bf16 elements per tile (512 threads x one 16-byte vector)


@pytest.fixture(scope="module")
def pkg():
    import sampling_topk_selection_amd as p

    p.load_library()
    yield p
    p.ds_topk_set_overrides(0, 0)


def _bf16(v):
    u = np.asarray(v, dtype=np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)  # round to nearest even


def _rows(n, seed):
    rng = np.random.default_rng(seed)
    levels = np.arange(-7.5, 8.0, 1.0, dtype=np.float32)  # 16 levels, exact in bf16
    ids = np.sort(rng.integers(0, 16, size=n))
    rows = [levels[ids], levels[ids[::-1]], rng.standard_normal(n).astype(np.float32)]
    r = rng.standard_normal(n).astype(np.float32)
    r[n // 3:] = -np.inf
    rows.append(r)
    rows.append(np.full(n, -2.5, dtype=np.float32))
    # rows pitched to 16 bytes; the padding holds NaN patterns past column n
    return pad_rows(np.stack([_bf16(x) for x in rows]), (n + 7) // 8 * 8)


@pytest.mark.parametrize("tiles", list(range(1, 10)))
def test_end_tiles_first(pkg, oracle_mod, tiles):
    for n in (tiles * TILE, tiles * TILE - 5):
        raw = _rows(n, seed=n)
        for k in (1025, 2048):
            st, oidx, oval = oracle_mod.topk(raw, "bf16", n, k, 1, True, nthreads=0)
            assert st == 0
            for segs in (1, 2):
                for tile_seed in (0, 0x2545F491):
                    log("visit order n=%d k=%d segs=%d tile_seed=%x" % (n, k, segs, tile_seed))
                    pkg.ds_topk_set_overrides(segs, tile_seed)
                    try:
                        gidx, gval = gpu_topk(raw, "bf16", n, k, 1, True)
                    finally:
                        pkg.ds_topk_set_overrides(0, 0)
                    assert_parity(raw, "bf16", n, k, 1, gidx, gval, oidx, oval,
                                  invariant_rows=range(raw.shape[0]))
