"""GPU: a seeded sweep over shapes and options -- dtype, batch, n, k, output
order, values, per-row lengths, index type, forced segment counts -- each
compared with the oracle (indices exactly when ordered, as sets otherwise;
values as bit copies)."""

import numpy as np
import pytest

from gpu_util import assert_parity, log, to_device, to_host_bits
from workloads import make_edge_rows

pytestmark = pytest.mark.gpu


def _cases(count=48, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(count):
        dtype = ["bf16", "f32"][c % 2]
        n = int(rng.choice([1, 3, 50, 64, 300, 2048, 2049, 5000, 40000, 150000]))
        k = int(min(n, rng.choice([1, 2, 7, 64, 300, 1024, 4096])))
        batch = int(rng.choice([1, 2, 5, 13]))
        out.append(dict(dtype=dtype, n=n, k=k, batch=batch, order=int(rng.integers(0, 3)),
                        retval=bool(rng.integers(0, 2)), levels=int(rng.choice([0, 0, 4, 40])),
                        lengths=bool(rng.integers(0, 4) == 0), i64=bool(rng.integers(0, 3) == 0),
                        segs=int(rng.choice([0, 0, 0, 1, 3])), seed=int(rng.integers(0, 1 << 30))))
    return out


@pytest.fixture(scope="module")
def pkg():
    import sampling_topk_selection_amd as p

    p.load_library()
    yield p
    p.ds_topk_set_overrides(0, 0)


@pytest.mark.parametrize("case", range(48))
def test_sweep(pkg, oracle_mod, case):
    import torch

    c = _cases()[case]
    log("sweep %d %s" % (case, c))
    raw = make_edge_rows(c["dtype"], c["batch"], c["n"], seed=c["seed"], levels=c["levels"], specials=0.02)
    rng = np.random.default_rng(c["seed"])
    lens = rng.integers(-2, c["n"] + 3, size=c["batch"]).tolist() if c["lengths"] else None
    x = to_device(raw, c["dtype"])
    pkg.ds_topk_set_overrides(c["segs"], 0)
    try:
        kw = dict(sorted_index=c["order"] == 1, sorted_value=c["order"] == 2, return_value=c["retval"], n=c["n"],
                  indices_type=torch.int64 if c["i64"] else torch.int32)
        if lens is not None:
            kw["lengths"] = torch.tensor(lens, dtype=torch.int32, device="cuda:0")
        val, idx = pkg.topk(x, c["k"], **kw)
    finally:
        pkg.ds_topk_set_overrides(0, 0)
    gidx = idx.cpu().numpy().astype(np.int64)
    gval = to_host_bits(val, c["dtype"]) if val is not None else None
    if lens is None:
        st, oidx, oval = oracle_mod.topk(raw, c["dtype"], c["n"], c["k"], c["order"], True, nthreads=0)
        assert st == 0
        assert_parity(raw, c["dtype"], c["n"], c["k"], c["order"], gidx.astype(np.int32), gval, oidx, oval)
    else:
        st, oidx, oval = oracle_mod.topk_lengths(raw, c["dtype"], c["n"], c["k"], lens, c["order"], True, nthreads=0)
        assert st == 0
        if c["order"]:
            assert np.array_equal(gidx, oidx)
            if gval is not None:
                assert np.array_equal(gval, oval)
        else:
            o, q = np.argsort(gidx, axis=1), np.argsort(oidx, axis=1)
            assert np.array_equal(np.take_along_axis(gidx, o, 1), np.take_along_axis(oidx, q, 1))
            if gval is not None:
                assert np.array_equal(np.take_along_axis(gval, o, 1), np.take_along_axis(oval, q, 1))
