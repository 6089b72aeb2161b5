"""GPU: ds_topk_sample (temperature, top-p, inverse-CDF draw over each row's
top-k) against the oracle.  The library sums fp32 weights; a draw that
falls within a few fp32 ulps of a boundary of the exact (double) sums may
take the neighbouring candidate, so such rows -- found from the double sums
-- accept either neighbour; all others must match exactly."""

import numpy as np
import pytest

from gpu_util import log, to_device
from workloads import make_edge_rows, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkg():
    import sampling_topk_selection_amd as p

    p.load_library()
    yield p


def _f64(vals, dtype):
    if dtype == "bf16":
        return (vals.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return vals.astype(np.float64)


def _allowed(oracle_mod, raw, dtype, n, k, T, P, U, tol=2e-5):
    """Per row: the oracle's token, and the candidate tokens a correct fp32
    draw may return (just the oracle's unless the draw is near a boundary)."""
    st, tok = oracle_mod.sample(raw, dtype, n, k, T, P, U)
    assert st == 0
    st, cidx, cval = oracle_mod.topk(raw, dtype, n, k, 2, True)
    assert st == 0
    allowed = []
    for r in range(raw.shape[0]):
        ok = {int(tok[r])}
        if T[r] > 0:
            x = _f64(cval[r], dtype)
            with np.errstate(invalid="ignore", over="ignore"):
                w = np.where(x == x[0], 1.0, np.where(np.isneginf(x), 0.0, np.exp((x - x[0]) / float(T[r]))))
            W = np.cumsum(w)
            j = int(np.nonzero(cidx[r] == tok[r])[0][0])
            band = tol * W[-1]
            near_p = np.min(np.abs(W - float(P[r]) * W[-1])) <= band
            mm = int(np.argmax(W >= float(P[r]) * W[-1])) if np.any(W >= float(P[r]) * W[-1]) else k - 1
            t = min(max(float(U[r]), 0.0), np.nextafter(1.0, 0.0)) * W[mm]
            near_t = np.min(np.abs(W[: mm + 1] - t)) <= band
            if near_p or near_t:
                lo, hi = max(0, j - 2), min(k, j + 3)
                ok |= set(int(c) for c in cidx[r, lo:hi])
        allowed.append(ok)
    return tok, allowed


def _check(pkg, oracle_mod, raw, dtype, n, k, T, P, U):
    import torch

    x = to_device(raw, dtype)
    t = torch.tensor(T, dtype=torch.float32, device="cuda:0")
    p = torch.tensor(P, dtype=torch.float32, device="cuda:0")
    u = torch.tensor(U, dtype=torch.float32, device="cuda:0")
    got = pkg.sample(x, k, t, p, u, n=n).cpu().numpy()
    tok, allowed = _allowed(oracle_mod, raw, dtype, n, k, T, P, U)
    exact = sum(1 for a in allowed if len(a) == 1)
    bad = [r for r in range(raw.shape[0]) if int(got[r]) not in allowed[r]]
    assert not bad, "rows %s: gpu %s, oracle %s" % (bad[:6], got[bad[:6]].tolist(), tok[bad[:6]].tolist())
    return exact


@pytest.mark.parametrize("cfg", ["C3", "C1"])
def test_sample_workload_rows(pkg, oracle_mod, cfg):
    w = make_workload(cfg)
    B = w.batch
    rng = np.random.default_rng(77)
    T = rng.uniform(0.3, 2.0, B).astype(np.float32)
    P = rng.uniform(0.2, 1.0, B).astype(np.float32)
    U = rng.random(B).astype(np.float32)
    log("sample %s batch=%d k=%d" % (cfg, B, w.k))
    exact = _check(pkg, oracle_mod, w.raw, w.dtype, w.n, w.k, T, P, U)
    assert exact >= B - max(2, B // 8)  # nearly every row is far from a boundary


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sample_edges(pkg, oracle_mod, dtype):
    # greedy (T <= 0, top_p 0, u 0), u near 1 and out of range, ties, +-inf
    n, k = 3000, 300
    raw = make_edge_rows(dtype, 8, n, seed=9, levels=12, specials=0.05)
    T = np.array([0.0, -1.0, 1.0, 1.0, 0.7, 5.0, 1.0, 1e-3], dtype=np.float32)
    P = np.array([1.0, 0.5, 0.0, 1.0, 0.9, 0.95, 1.5, 1.0], dtype=np.float32)
    U = np.array([0.5, 0.5, 0.9, 0.0, 0.999999, 1.5, -0.2, 0.3], dtype=np.float32)
    log("sample edges %s" % dtype)
    _check(pkg, oracle_mod, raw, dtype, n, k, T, P, U)


@pytest.mark.parametrize("dtype,n,k,segs,levels", [
    ("f32", 1500, 100, 0, 0),     # one wave per row, then the sampling kernel
    ("bf16", 40000, 2000, 0, 0),  # k > 1024: the sampling kernel after the selection
    ("f32", 20000, 700, 0, 7),    # drawn in the selection's launch, k above one entry per thread
    ("bf16", 9000, 1024, 0, 0),   # the largest k drawn in the selection's launch
    ("bf16", 60000, 300, 3, 0),   # split rows: the merging workgroup draws
    ("f32", 60000, 700, 4, 5),    # split rows, k above one entry per thread
])
def test_sample_paths(pkg, oracle_mod, dtype, n, k, segs, levels):
    B = 6
    raw = make_edge_rows(dtype, B, n, seed=n + k, levels=levels, specials=0.0)
    rng = np.random.default_rng(n * 7 + k)
    T = rng.uniform(0.2, 3.0, B).astype(np.float32)
    T[0] = 0.0  # greedy
    P = rng.uniform(0.3, 1.0, B).astype(np.float32)
    U = rng.random(B).astype(np.float32)
    log("sample path %s n=%d k=%d segs=%d levels=%d" % (dtype, n, k, segs, levels))
    pkg.ds_topk_set_overrides(segs, 0, 0)
    try:
        _check(pkg, oracle_mod, raw, dtype, n, k, T, P, U)
    finally:
        pkg.ds_topk_set_overrides(0, 0, 0)


def test_sample_nan_is_reported(pkg):
    import torch

    raw = make_edge_rows("f32", 2, 512, seed=3)
    raw[1, 100] = np.nan
    with pytest.raises(FloatingPointError):
        pkg.sample(to_device(raw, "f32"), 16, 1.0, 0.9, 0.5, n=512)
    torch.cuda.synchronize()
