"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself:
  * brute-force rank counting (pure Python loops, and a numpy broadcast form);
  * closed forms: strictly ascending rows, constant rows, k = n, rows whose
    valid prefix is shorter than k (-inf tail), quantised ascending levels;
  * a library cross-check (numpy argpartition) on rows without ties;
  * the O(n) completeness invariant at the full workload sizes;
  * bit-exact values, ascending sorted indices, NaN status, argument errors;
  * planted mistakes: mutated copies of oracle.c must fail these pins.
"""

import math
import os
import subprocess
import tempfile

import numpy as np
import pytest

import brute
from brute import topk_set_loop, topk_set_numpy
from invariants import check_topk_row, check_values_row
from workloads import CONFIGS, bf16_bits_from_f32, make_edge_rows, make_workload

DTYPES = ["bf16", "f32"]


def _oracle_set(oracle_mod, raw, dtype, n, k):
    st, idx, _ = oracle_mod.topk(raw, dtype, n, k, sorted_index=True, return_value=False)
    assert st == oracle_mod.OK
    return idx


@pytest.mark.parametrize("dtype", DTYPES)
def test_brute_loop_tiny_every_k(oracle_mod, dtype):
    # Tiny rows with heavy ties, +-0, +-inf, denormals; every k in 1..n.
    for seed in range(40):
        n = 1 + seed % 23
        raw = make_edge_rows(dtype, 1, n, seed=seed, levels=3 + seed % 4, specials=0.3)
        for k in range(1, n + 1):
            got = _oracle_set(oracle_mod, raw, dtype, n, k)[0]
            want = topk_set_loop(raw[0, :n], dtype, k)
            assert got.tolist() == want, (seed, n, k)


@pytest.mark.parametrize("dtype", DTYPES)
def test_brute_numpy_medium(oracle_mod, dtype):
    rng = np.random.default_rng(123)
    for seed in range(12):
        n = int(rng.integers(50, 2049))
        k = int(rng.integers(1, min(n, 4096) + 1))
        raw = make_edge_rows(dtype, 2, n, seed=100 + seed, levels=[0, 5, 40][seed % 3],
                             specials=[0.0, 0.05, 0.5][seed % 3])
        got = _oracle_set(oracle_mod, raw, dtype, n, k)
        for r in range(2):
            want = topk_set_numpy(raw[r, :n], dtype, k)
            assert got[r].tolist() == want.tolist(), (seed, n, k, r)


def test_brute_forms_agree():
    # The two brute-force forms must agree with each other.
    raw = make_edge_rows("bf16", 3, 30, seed=7, levels=4, specials=0.4)
    for r in range(3):
        for k in (1, 5, 17, 30):
            assert topk_set_loop(raw[r, :30], "bf16", k) == topk_set_numpy(raw[r, :30], "bf16", k).tolist()


@pytest.mark.parametrize("dtype", DTYPES)
def test_closed_form_ascending(oracle_mod, dtype):
    # Strictly ascending distinct values: the top-k is the last k columns.
    n, k = 1000, 77
    if dtype == "bf16":
        neg = np.arange(0xBF80 + n // 2 - 1, 0xBF80 - 1, -1)  # -big ... -1.0
        pos = np.arange(0x3F80, 0x3F80 + n - n // 2)         # +1.0 ... +big
        raw = np.concatenate([neg, pos]).astype(np.uint16)[None]
    else:
        raw = np.linspace(-50, 50, n).astype(np.float32)[None]
        assert np.all(np.diff(raw[0]) > 0)
    got = _oracle_set(oracle_mod, raw, dtype, n, k)[0]
    assert got.tolist() == list(range(n - k, n))


@pytest.mark.parametrize("dtype", DTYPES)
def test_closed_form_constant(oracle_mod, dtype):
    n = 513
    for v in (1.5, 0.0, -0.0, float("inf"), float("-inf")):
        raw = (bf16_bits_from_f32(np.full(n, v, np.float32))[None] if dtype == "bf16"
               else np.full((1, n), v, np.float32))
        for k in (1, 64, n):
            got = _oracle_set(oracle_mod, raw, dtype, n, k)[0]
            assert got.tolist() == list(range(k)), (v, k)


@pytest.mark.parametrize("dtype", DTYPES)
def test_closed_form_k_equals_n(oracle_mod, dtype):
    raw = make_edge_rows(dtype, 3, 257, seed=9, specials=0.2)
    st, idx, val = oracle_mod.topk(raw, dtype, 257, 257, sorted_index=True, return_value=True)
    assert st == 0
    for r in range(3):
        assert idx[r].tolist() == list(range(257))
        check_values_row(raw[r], idx[r], val[r])


def test_closed_form_short_valid_prefix(oracle_mod):
    # A valid prefix of length L < k followed by -inf: the answer is {0..k-1}
    # (all L valid entries, then the lowest-index -inf entries).
    n, k = 4096, 512
    rng = np.random.default_rng(5)
    for L in (1, 100, 511, 512):
        row = bf16_bits_from_f32(rng.standard_normal(n).astype(np.float32))
        row[L:] = 0xFF80
        got = _oracle_set(oracle_mod, row[None], "bf16", n, k)[0]
        assert got.tolist() == list(range(k)), L


def c5_closed_form(level_counts, k):
    """Top-k of a row of ascending quantised levels, ties to lower index."""
    counts = np.asarray(level_counts)
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    above = 0
    for lvl in range(len(counts) - 1, -1, -1):
        if above + counts[lvl] >= k:
            take = k - above
            tied = np.arange(starts[lvl], starts[lvl] + take)
            rest = np.arange(starts[lvl] + counts[lvl], counts.sum())
            return np.concatenate([tied, rest])
        above += counts[lvl]
    raise AssertionError


def test_closed_form_quantised_ascending(oracle_mod):
    w = make_workload("C5", batch=16)
    st, idx, val = oracle_mod.topk(w.raw, "bf16", w.n, w.k, True, True, nthreads=0)
    assert st == 0
    for r in range(w.batch):
        assert idx[r].tolist() == c5_closed_form(w.meta["level_counts"][r], w.k).tolist()
        check_values_row(w.raw[r], idx[r], val[r])


def test_library_crosscheck_no_ties(oracle_mod):
    # Distinct fp32 values in shuffled order: no ties, so numpy's
    # argpartition gives the same set.
    rng = np.random.default_rng(11)
    x = ((rng.permuted(np.tile(np.arange(20000), (8, 1)), axis=1) - 10000) * 0.5).astype(np.float32)
    assert all(np.unique(r).size == r.size for r in x)
    for k in (1, 100, 4096):
        got = _oracle_set(oracle_mod, x, "f32", 20000, k)
        for r in range(8):
            want = np.sort(np.argpartition(-x[r].astype(np.float64), k - 1)[:k])
            assert got[r].tolist() == want.tolist()


@pytest.mark.parametrize("cfg", sorted(CONFIGS))
def test_full_workloads_invariant(oracle_mod, cfg):
    w = make_workload(cfg)
    st, idx, val = oracle_mod.topk(w.raw, w.dtype, w.n, w.k, w.sorted_index, True, nthreads=0)
    assert st == 0
    rows = range(w.batch) if w.batch <= 8 else range(0, w.batch, max(1, w.batch // 8))
    for r in rows:
        check_topk_row(w.raw[r], w.dtype, w.n, w.k, idx[r], sorted_index=w.sorted_index)
        check_values_row(w.raw[r], idx[r], val[r])


@pytest.mark.parametrize("dtype", DTYPES)
def test_nan_status(oracle_mod, dtype):
    n = 100
    raw = make_edge_rows(dtype, 3, n, seed=1, row_stride=104)
    # padding (columns n..row_stride) already holds NaN: must be ignored
    st, _, _ = oracle_mod.topk(raw, dtype, n, 10)
    assert st == oracle_mod.OK
    nan_bits = [0x7FC0, 0xFFC0, 0x7F81, 0xFF81] if dtype == "bf16" else [
        np.uint32(0x7FC00000).view(np.float32), np.uint32(0xFFC00000).view(np.float32),
        np.uint32(0x7F800001).view(np.float32), np.uint32(0xFF800001).view(np.float32)]
    for b in nan_bits:
        for col in (0, n // 2, n - 1):
            bad = raw.copy()
            bad[2, col] = b
            st, _, _ = oracle_mod.topk(bad, dtype, n, 10)
            assert st == oracle_mod.NAN, (repr(b), col)


def test_bad_args(oracle_mod):
    raw = make_edge_rows("f32", 2, 16, seed=0)
    assert oracle_mod.topk(raw, "f32", 16, 0)[0] == oracle_mod.BAD_ARG
    assert oracle_mod.topk(raw, "f32", 16, 17)[0] == oracle_mod.BAD_ARG
    assert oracle_mod.topk(raw, "f32", 17, 4)[0] == oracle_mod.BAD_ARG  # row_stride < n


def test_unsorted_is_rank_order(oracle_mod):
    raw = make_edge_rows("bf16", 1, 300, seed=3, levels=6)
    st, a, _ = oracle_mod.topk(raw, "bf16", 300, 40, sorted_index=True)
    st2, b, _ = oracle_mod.topk(raw, "bf16", 300, 40, sorted_index=False)
    assert st == st2 == 0
    assert sorted(b[0].tolist()) == a[0].tolist()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_value_order_is_rank_order(oracle_mod, dtype):
    # Order 2 lists the selection by value: the j-th output has brute-force
    # rank j (ties by lower index, +0 before -0), checked position by position.
    for seed in range(6):
        n = 40 + 13 * seed
        raw = make_edge_rows(dtype, 1, n, seed=100 + seed, levels=5 if seed % 2 else 0, specials=0.1)
        vals = brute.decode(raw[0, :n], dtype)
        ranks = [sum(1 for j in range(n) if j != i and brute.precedes(vals[j], j, vals[i], i)) for i in range(n)]
        by_rank = sorted(range(n), key=lambda i: ranks[i])
        for k in (1, 7, n // 2, n):
            st, idx, val = oracle_mod.topk(raw, dtype, n, k, sorted_index=2)
            assert st == 0
            assert idx[0].tolist() == by_rank[:k]
            assert np.array_equal(val[0], raw[0, idx[0]])
    assert oracle_mod.topk(make_edge_rows("f32", 1, 16, seed=0), "f32", 16, 4, sorted_index=3)[0] == oracle_mod.BAD_ARG


def _neg_inf_tail(raw, dtype, lens):
    # the rows as the lengths describe them: columns >= len hold -inf
    t = raw.copy()
    ninf = np.uint16(0xFF80) if dtype == "bf16" else np.float32(-np.inf)
    for r, L in enumerate(lens):
        t[r, max(0, min(L, t.shape[1])):] = ninf
    return t


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lengths_match_brute_force_on_neg_inf_tails(oracle_mod, dtype):
    # Row r with valid length L is the row whose columns >= L are -inf: the
    # selected set is checked against brute-force ranks of that row, the value
    # order position by position, and the tail's values are -inf bit patterns.
    rng = np.random.default_rng(7)
    for trial in range(8):
        n = int(rng.integers(20, 90))
        raw = make_edge_rows(dtype, 4, n, seed=200 + trial, levels=4 if trial % 2 else 0, specials=0.05)
        lens = [0, int(rng.integers(1, n)), n, n + 5][: raw.shape[0]]
        filled = _neg_inf_tail(raw, dtype, lens)
        for k in (1, 5, n):
            st, idx, val = oracle_mod.topk_lengths(raw, dtype, n, k, lens, sorted_index=2)
            assert st == 0
            for r in range(raw.shape[0]):
                row = filled[r, :n]
                assert sorted(idx[r].tolist()) == topk_set_loop(row, dtype, k)
                vals = brute.decode(row, dtype)
                ranks = [sum(1 for j in range(n) if j != i and brute.precedes(vals[j], j, vals[i], i))
                         for i in range(n)]
                assert idx[r].tolist() == sorted(range(n), key=lambda i: ranks[i])[:k]
                want = filled[r, idx[r]]
                assert np.array_equal(val[r].view(np.uint16 if dtype == "bf16" else np.uint32),
                                      want.view(np.uint16 if dtype == "bf16" else np.uint32))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lengths_never_read_the_tail(oracle_mod, dtype):
    # NaN past a row's length is not looked at; NaN inside it is reported.
    n = 64
    raw = make_edge_rows(dtype, 2, n, seed=5)
    nan = np.uint16(0x7FC1) if dtype == "bf16" else np.float32(np.nan)
    raw[:, 40:] = nan
    st, idx, _ = oracle_mod.topk_lengths(raw, dtype, n, 8, [40, 12], sorted_index=1)
    assert st == 0
    assert oracle_mod.topk_lengths(raw, dtype, n, 8, [41, 12], sorted_index=1)[0] == oracle_mod.NAN
    # a length below k: the valid columns, then the first tail columns
    st, idx, val = oracle_mod.topk_lengths(raw, dtype, n, 8, [3, 0], sorted_index=1)
    assert st == 0 and idx[0].tolist() == list(range(8)) and idx[1].tolist() == list(range(8))


# ---------------------------------------------------------------- sampling over the top-k
def _row(dtype, vals, n=64, fill=-1000.0):
    # one row: the given leading values, then a low fill
    x = np.full((1, n), fill, dtype=np.float32)
    x[0, : len(vals)] = vals
    return bf16_bits_from_f32(x) if dtype == "bf16" else x


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sample_greedy_cases(oracle_mod, dtype):
    # T <= 0, top_p = 0 and u = 0 all give the first candidate in value order
    raw = make_edge_rows(dtype, 3, 500, seed=31)
    st, top, _ = oracle_mod.topk(raw, dtype, 500, 1, 2, False)
    for T, p, u in ((0.0, 1.0, 0.7), (1.0, 0.0, 0.7), (1.0, 1.0, 0.0), (-1.0, 0.5, 0.5)):
        st, tok = oracle_mod.sample(raw, dtype, 500, 50, T, p, u)
        assert st == 0 and tok.tolist() == top[:, 0].tolist()


def test_sample_equal_candidates_inverse_cdf(oracle_mod):
    # k equal top values: uniform weights, token = the (floor(u k) + 1)-th
    # lowest index among them
    cols = [3, 9, 10, 17, 40]
    x = np.full((1, 64), -5.0, dtype=np.float32)
    x[0, cols] = 2.0
    for u in (0.0, 0.19, 0.2, 0.5, 0.79, 0.8, 0.99):
        st, tok = oracle_mod.sample(x, "f32", 64, 5, 1.0, 1.0, u)
        assert st == 0 and tok[0] == cols[int(u * 5)]
    # u exactly on a step (W_j = j, u k = j in binary): the draw is the next one
    x[0, cols[4]] = -5.0
    for u in (0.25, 0.5, 0.75):
        st, tok = oracle_mod.sample(x, "f32", 64, 4, 1.0, 1.0, u)
        assert st == 0 and tok[0] == cols[int(u * 4)]
    # top_p exactly on a step (W_2 = 2 = 0.5 W_4): the nucleus keeps two, so
    # u = 0.9 draws at t = 1.8, the second
    st, tok = oracle_mod.sample(x, "f32", 64, 4, 1.0, 0.5, 0.9)
    assert st == 0 and tok[0] == cols[1]


@pytest.mark.parametrize("T", [0.5, 1.0, 3.0])
def test_sample_two_candidates_analytic(oracle_mod, T):
    # p(first) = 1 / (1 + exp((b - a) / T)); the fill is exp(-1000 / T) = 0
    a, b = 1.25, 0.5
    p1 = 1.0 / (1.0 + math.exp((b - a) / T))
    x = _row("f32", [b, a])  # the larger value at column 1
    for u, want in ((p1 - 1e-6, 1), (p1 + 1e-6, 0)):
        st, tok = oracle_mod.sample(x, "f32", 64, 8, T, 1.0, u)
        assert st == 0 and tok[0] == want


def test_sample_nucleus_closed_form(oracle_mod):
    # weights 1, 1/2, 1/4 (logits 0, -ln 2, -ln 4 at T = 1): W = 1, 1.5, 1.75;
    # top_p 0.8 keeps two (1.5 >= 1.4), so u = 0.9 -> t = 1.35 -> second,
    # u = 0.6 -> t = 0.9 -> first; top_p 0.5 keeps one; top_p 1 keeps all
    # three: u = 0.9 -> t = 1.575 -> third, 0.6 -> 1.05 -> second,
    # 0.5 -> 0.875 -> first
    x = _row("f32", [0.0, -math.log(2.0), -math.log(4.0)])
    cases = ((0.8, 0.9, 1), (0.8, 0.6, 0), (0.5, 0.99, 0), (1.0, 0.9, 2), (1.0, 0.6, 1), (1.0, 0.5, 0))
    for p, u, want in cases:
        st, tok = oracle_mod.sample(x, "f32", 64, 3, 1.0, p, u)
        assert st == 0 and tok[0] == want, (p, u)


def test_sample_frequencies_follow_softmax(oracle_mod):
    # u on a uniform grid: each candidate is drawn in proportion to its
    # nucleus-normalised softmax weight (to within one grid step)
    vals = [1.0, 0.7, 0.2, -0.3, -1.1, -2.0]
    x = _row("f32", vals)
    T, p, N = 0.8, 0.9, 2000
    w = np.exp((np.array(vals) - vals[0]) / T)
    W = np.cumsum(w)
    m = int(np.argmax(W >= p * W[-1])) + 1
    want = w[:m] / W[m - 1] * N
    grid = (np.arange(N) + 0.5) / N
    xs = np.repeat(x, N, axis=0)
    st, tok = oracle_mod.sample(xs, "f32", 64, 6, T, p, grid)
    assert st == 0
    counts = np.bincount(tok, minlength=64)[: len(vals)]
    assert np.all(np.abs(counts[:m] - want) <= 1.0) and counts[m:].sum() == 0


def test_sample_infinite_tops(oracle_mod):
    # two +inf share the mass (lower index first); -inf candidates get none
    x = np.full((1, 64), -np.inf, dtype=np.float32)
    x[0, 20] = np.inf
    x[0, 7] = np.inf
    x[0, 30] = 5.0
    for u, want in ((0.1, 7), (0.49, 7), (0.51, 20), (0.99, 20)):
        st, tok = oracle_mod.sample(x, "f32", 64, 10, 1.0, 1.0, u)
        assert st == 0 and tok[0] == want


# ---------------------------------------------------------------- planted mistakes
_MUTANTS = {
    "tie_to_higher_index": ("if (a->i < b->i) return -1;\n    if (a->i > b->i) return 1;",
                            "if (a->i > b->i) return -1;\n    if (a->i < b->i) return 1;"),
    "zero_sign_reversed": ("return sa ? 1 : -1;", "return sa ? -1 : 1;"),
    "drops_last_column": ("for (int64_t c = 0; c < n; ++c) {", "for (int64_t c = 0; c < n - 1; ++c) {"),
    "bf16_low_half": ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b;"),
    "no_nan_check": ("if (isnan(it[c].v)) {", "if (0) {"),
    "value_order_by_index": ("if (sorted_index == 1) qsort", "if (sorted_index) qsort"),
    "lengths_read_tail": ("it[c].v = c < len ? widen(row, dtype, c) : -INFINITY;", "it[c].v = widen(row, dtype, c);"),
    "lengths_off_by_one": ("it[c].v = c < len ? widen", "it[c].v = c <= len ? widen"),
    "sample_ignores_temperature": ("exp((x - x1) / T)", "exp(x - x1)"),
    "sample_nucleus_strict": ("if (W[j] >= p * W[k - 1]) {", "if (W[j] > p * W[k - 1]) {"),
    "sample_draw_not_strict": ("if (W[j] > t) {", "if (W[j] >= t) {"),
}


def _build_mutant(name):
    src = open(os.path.join(os.path.dirname(__file__), "..", "oracle", "oracle.c")).read()
    old, new = _MUTANTS[name]
    assert old in src, name
    d = tempfile.mkdtemp()
    cpath, so = os.path.join(d, "m.c"), os.path.join(d, "libm.so")
    open(cpath, "w").write(src.replace(old, new))
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", so, cpath, "-lm"])
    return so


def _pins_pass(oracle_mod):
    try:
        test_brute_loop_tiny_every_k(oracle_mod, "bf16")
        test_brute_loop_tiny_every_k(oracle_mod, "f32")
        test_closed_form_ascending(oracle_mod, "bf16")
        test_closed_form_constant(oracle_mod, "bf16")
        test_nan_status(oracle_mod, "bf16")
        test_nan_status(oracle_mod, "f32")
        test_value_order_is_rank_order(oracle_mod, "bf16")
        test_lengths_match_brute_force_on_neg_inf_tails(oracle_mod, "f32")
        test_lengths_never_read_the_tail(oracle_mod, "bf16")
        test_sample_greedy_cases(oracle_mod, "f32")
        test_sample_equal_candidates_inverse_cdf(oracle_mod)
        test_sample_two_candidates_analytic(oracle_mod, 0.5)
        test_sample_nucleus_closed_form(oracle_mod)
        test_sample_frequencies_follow_softmax(oracle_mod)
        test_sample_infinite_tops(oracle_mod)
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("name", sorted(_MUTANTS))
def test_planted_mistake_is_caught(oracle_mod, name, monkeypatch):
    import ctypes

    so = _build_mutant(name)
    lib = ctypes.CDLL(so)
    lib.oracle_topk.restype = ctypes.c_int
    lib.oracle_topk.argtypes = oracle_mod._load().oracle_topk.argtypes
    lib.oracle_topk_lengths.restype = ctypes.c_int
    lib.oracle_topk_lengths.argtypes = oracle_mod._load().oracle_topk_lengths.argtypes
    lib.oracle_sample.restype = ctypes.c_int
    lib.oracle_sample.argtypes = oracle_mod._load().oracle_sample.argtypes
    monkeypatch.setattr(oracle_mod, "_lib", lib)
    assert not _pins_pass(oracle_mod), "pins did not catch mutant %s" % name
