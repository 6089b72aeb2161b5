"""GPU edge cases against the oracle: ragged lengths with NaN in the padding,
k at the ends of its range, k = n, ties everywhere, +-0, +-inf, denormals,
NaN detection, both plans, the async entry point and run-to-run stability."""

import numpy as np
import pytest

from gpu_util import assert_parity, gpu_topk, log, to_device
from workloads import make_edge_rows

pytestmark = pytest.mark.gpu

DTYPES = ["bf16", "f32"]


@pytest.fixture(scope="module")
def pkg():
    import sampling_topk_selection_amd as p

    p.load_library()
    yield p
    p.ds_topk_set_overrides(0, 0)


def _check(pkg, oracle_mod, raw, dtype, n, k, sorted_index, segs=0, retval=True):
    pkg.ds_topk_set_overrides(segs, 0)
    try:
        gidx, gval = gpu_topk(raw, dtype, n, k, sorted_index, retval)
    finally:
        pkg.ds_topk_set_overrides(0, 0)
    st, oidx, oval = oracle_mod.topk(raw, dtype, n, k, sorted_index, True, nthreads=0)
    assert st == 0
    assert_parity(raw, dtype, n, k, sorted_index, gidx, gval, oidx, oval,
                  invariant_rows=range(raw.shape[0]))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n", [1, 7, 9, 100, 1001, 4097, 70001])
@pytest.mark.parametrize("segs", [0, 1, 5])
def test_ragged_lengths_nan_padding(pkg, oracle_mod, dtype, n, segs):
    # row pitch padded to 16 bytes, padding filled with NaN (must be ignored)
    raw = make_edge_rows(dtype, 3, n, seed=n, specials=0.02)
    log("ragged %s n=%d segs=%d pitch=%d" % (dtype, n, segs, raw.shape[1]))
    for k in sorted({1, min(n, 5), min(n, 64), min(n, 4096)}):
        for srt in (True, False):
            _check(pkg, oracle_mod, raw, dtype, n, k, srt, segs)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k", [1, 2, 63, 64, 65, 511, 1024, 1025, 4095, 4096])
def test_k_range(pkg, oracle_mod, dtype, k):
    n = 40000
    raw = make_edge_rows(dtype, 2, n, seed=k, levels=0)
    log("k-range %s k=%d" % (dtype, k))
    for segs in (0, 1, 4):
        _check(pkg, oracle_mod, raw, dtype, n, k, True, segs)
        _check(pkg, oracle_mod, raw, dtype, n, k, False, segs, retval=False)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("levels", [1, 2, 3, 16])
def test_heavy_ties_and_specials(pkg, oracle_mod, dtype, levels):
    raw = make_edge_rows(dtype, 4, 30000, seed=levels, levels=levels, specials=0.1)
    log("ties %s levels=%d" % (dtype, levels))
    for k in (1, 100, 3000, 4096):
        for segs in (0, 1, 7):
            _check(pkg, oracle_mod, raw, dtype, 30000, k, True, segs)


@pytest.mark.parametrize("dtype", DTYPES)
def test_constant_rows_and_zero_signs(pkg, oracle_mod, dtype):
    n = 9000
    rows = []
    for bits in ([0x0000, 0x8000] if dtype == "bf16" else [0x00000000, 0x80000000]):
        rows.append(np.full(n, bits, dtype=np.uint16 if dtype == "bf16" else np.uint32))
    mixed = np.where(np.arange(n) % 3 == 0, rows[1], rows[0])  # -0 and +0 interleaved
    raw = np.stack(rows + [mixed])
    if dtype == "f32":
        raw = raw.view(np.float32)
    log("zeros %s" % dtype)
    for k in (1, 3000, 4096):
        for segs in (0, 1, 3):
            _check(pkg, oracle_mod, raw, dtype, n, k, True, segs)


@pytest.mark.parametrize("dtype", DTYPES)
def test_infinities_and_short_valid_prefix(pkg, oracle_mod, dtype):
    n, k = 20000, 512
    raw = make_edge_rows(dtype, 6, n, seed=77)
    ninf = 0xFF80 if dtype == "bf16" else np.float32(-np.inf)
    pinf = 0x7F80 if dtype == "bf16" else np.float32(np.inf)
    for r, L in enumerate([1, 100, 511, 512, 513, 19999]):
        raw[r, L:n] = ninf
    raw[5, 17] = pinf
    raw[5, 3] = pinf
    log("inf %s" % dtype)
    for segs in (0, 1, 6):
        _check(pkg, oracle_mod, raw, dtype, n, k, True, segs)
        _check(pkg, oracle_mod, raw, dtype, n, k, False, segs)


@pytest.mark.parametrize("dtype", DTYPES)
def test_many_short_rows(pkg, oracle_mod, dtype):
    raw = make_edge_rows(dtype, 1500, 300, seed=5, levels=20)
    log("many rows %s" % dtype)
    _check(pkg, oracle_mod, raw, dtype, 300, 32, True)
    _check(pkg, oracle_mod, raw, dtype, 300, 32, False)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("segs", [0, 1, 4])
def test_nan_detection(pkg, dtype, segs):
    import sampling_topk_selection_amd as p

    n = 5001
    raw = make_edge_rows(dtype, 3, n, seed=3)  # padding holds NaN: ignored
    nan_patterns = ([0x7FC0, 0xFFC0, 0x7F81, 0xFF81] if dtype == "bf16" else
                    [np.uint32(b).view(np.float32) for b in (0x7FC00000, 0xFFC00000, 0x7F800001, 0xFF800001)])
    log("nan %s segs=%d" % (dtype, segs))
    p.ds_topk_set_overrides(segs, 0)
    try:
        p.topk(to_device(raw, dtype), 10, n=n)  # padding NaN only: fine
        for b in nan_patterns:
            for col in (0, n // 2, n - 1):
                bad = raw.copy()
                bad[1, col] = b
                with pytest.raises(FloatingPointError):
                    p.topk(to_device(bad, dtype), 10, n=n)
        # a clean call after a NaN call must succeed again
        p.topk(to_device(raw, dtype), 10, n=n)
    finally:
        p.ds_topk_set_overrides(0, 0)


def test_async_entry_point_and_status(pkg, oracle_mod):
    import torch

    n, k = 50000, 256
    raw = make_edge_rows("f32", 5, n, seed=9)
    x = to_device(raw, "f32")
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    outs = [pkg.topk_async(x, k, status, sorted_index=True) for _ in range(3)]
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    st, oidx, oval = oracle_mod.topk(raw, "f32", n, k, True, True)
    for val, idx in outs:
        assert np.array_equal(idx.cpu().numpy(), oidx)
        assert np.array_equal(val.cpu().numpy().view(np.uint32), oval.view(np.uint32))
    bad = raw.copy()
    bad[2, 1234] = np.float32(np.nan)
    pkg.topk_async(to_device(bad, "f32"), k, status)
    torch.cuda.synchronize()
    assert int(status.item()) == pkg.DS_ERR_NAN


def test_side_stream_ordering(pkg, oracle_mod):
    import torch

    n, k = 129280, 512
    raw = make_edge_rows("f32", 8, n, seed=21)
    st, oidx, _ = oracle_mod.topk(raw, "f32", n, k, True, False, nthreads=0)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        x = to_device(raw, "f32")
        x.add_(0.0)
        _, idx = pkg.topk(x, k, sorted_index=True, return_value=False)
    assert np.array_equal(idx.cpu().numpy(), oidx)


@pytest.mark.parametrize("cfg", ["C2", "C3", "C5"])
def test_repeatability(pkg, cfg):
    from workloads import make_workload

    w = make_workload(cfg, batch=8)
    x = to_device(w.raw, w.dtype)
    log("repeat %s" % cfg)
    ref = None
    for rep in range(12):
        if rep == 6:
            pkg.ds_topk_set_overrides(0, 12345)  # another tile order: same answer
        val, idx = pkg.topk(x, w.k, sorted_index=True, return_value=True, n=w.n)
        cur = idx.cpu().numpy()
        if ref is None:
            ref = cur
        assert np.array_equal(cur, ref)
        _, uidx = pkg.topk(x, w.k, sorted_index=False, return_value=False, n=w.n)
        assert np.array_equal(np.sort(uidx.cpu().numpy(), axis=1), ref)
    pkg.ds_topk_set_overrides(0, 0)


def test_repeated_calls_overflow_path(pkg, oracle_mod):
    """The full ragged-decode workload (rows whose -inf tails fill whole
    segments, so candidate buffers overflow and tiles are filtered again),
    called back to back: every call returns DS_OK and the oracle's sets."""
    from workloads import make_workload

    w = make_workload("C4")
    st, oidx, _ = oracle_mod.topk(w.raw, w.dtype, w.n, w.k, False, False, nthreads=0)
    assert st == 0
    want = np.sort(oidx, axis=1)
    x = to_device(w.raw, w.dtype)
    log("repeated C4 calls")
    for rep in range(20):
        val, idx = pkg.topk(x, w.k, sorted_index=False, return_value=True, n=w.n)
        got = np.sort(idx.cpu().numpy(), axis=1)
        bad = np.nonzero(np.any(got != want, axis=1))[0]
        assert bad.size == 0, "call %d: rows %s differ" % (rep, bad[:8].tolist())


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n", [16384, 16385, 65536, 65537, 262144, 262145])
def test_index_order_paths(pkg, oracle_mod, dtype, n):
    # Index order from the column bitmap at each row width of its table
    # (one word per thread up to 16384 columns, then 2, 4, ... words), and
    # from the bitonic sort: forced, and where the table does not fit.
    raw = make_edge_rows(dtype, 2, n, seed=n + 3, levels=64 if dtype == "bf16" else 0)
    for k in (1, 300, 4096):
        st, oidx, oval = oracle_mod.topk(raw, dtype, n, k, True, True, nthreads=0)
        assert st == 0
        for segs in (1, 3):
            for flags in (0, 1):
                log("index order %s n=%d k=%d segs=%d flags=%d" % (dtype, n, k, segs, flags))
                pkg.ds_topk_set_overrides(segs, 0, flags)
                try:
                    gidx, gval = gpu_topk(raw, dtype, n, k, True, True)
                finally:
                    pkg.ds_topk_set_overrides(0, 0, 0)
                assert_parity(raw, dtype, n, k, True, gidx, gval, oidx, oval, invariant_rows=range(raw.shape[0]))



@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("levels", [0, 3, 64])
def test_value_order_edges(pkg, oracle_mod, dtype, levels):
    # Value order through every path: short and long rows, ties, +-0, +-inf,
    # one segment and several, k up to 4096.
    for n in (1, 9, 1001, 70001):
        raw = make_edge_rows(dtype, 3, n, seed=n + levels, levels=levels, specials=0.05)
        for k in sorted({1, min(n, 33), min(n, 4096)}):
            log("value order %s levels=%d n=%d k=%d" % (dtype, levels, n, k))
            for segs in (0, 1, 4):
                _check(pkg, oracle_mod, raw, dtype, n, k, 2, segs)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("levels", [0, 3])
def test_value_order_rank_sizes(pkg, oracle_mod, dtype, levels):
    # Value order for k up to the workgroup size ranks each wave's entries as
    # one run of 64: k just below, at and above a run boundary and at the
    # largest such k, through one workgroup per row and through the merge.
    n = 20011
    raw = make_edge_rows(dtype, 4, n, seed=77 + levels, levels=levels, specials=0.02)
    for k in (63, 64, 65, 129, 448, 511, 512, 513):
        log("value order ranks %s levels=%d k=%d" % (dtype, levels, k))
        for segs in (0, 1, 4):
            _check(pkg, oracle_mod, raw, dtype, n, k, 2, segs)


@pytest.mark.parametrize("cfg", ["C3", "C2"])
def test_async_call_in_a_graph(pkg, oracle_mod, cfg):
    # ds_topk_async captured in a HIP graph (after a warm-up call sized the
    # workspace) and replayed several times, with eager calls in between:
    # every replay gives the eager answer.
    import torch

    from workloads import make_workload

    w = make_workload(cfg, batch=8)
    x = to_device(w.raw, w.dtype)
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    log("graph replay %s" % cfg)
    ref_v, ref_i = pkg.topk(x, w.k, sorted_index=True, return_value=True, n=w.n)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out_v = torch.empty_like(ref_v)
        out_i = torch.empty_like(ref_i)
        pkg.topk_async(x, w.k, status, sorted_index=True, n=w.n, out=(out_v, out_i))  # warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pkg.topk_async(x, w.k, status, sorted_index=True, n=w.n, out=(out_v, out_i))
    for rep in range(4):
        out_i.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_i, ref_i) and torch.equal(out_v, ref_v), "replay %d" % rep
        pkg.topk(x, w.k, sorted_index=False, return_value=False, n=w.n)  # eager work between replays
    assert int(status.item()) == 0
