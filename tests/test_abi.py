"""The C-ABI library without a GPU: it loads, exports every declared symbol,
and its host-side checks and planning behave as documented.  None of these
calls reaches the GPU (argument errors return before any HIP call)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ds_topk.h")


@pytest.fixture(scope="module")
def pkg():
    from sampling_topk_selection_amd import build as b

    b.build(force=False)
    import sampling_topk_selection_amd as p

    p.load_library()
    return p


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ds_topk\w*)\s*\(", src)))


def test_header_declares_the_boundary():
    fns = declared_functions()
    assert "ds_topk" in fns and "ds_topk_status_string" in fns
    assert len(fns) >= 5


def test_library_exports_every_declared_symbol(pkg):
    lib = ctypes.CDLL(pkg.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), "missing export %s" % name
    assert set(pkg.EXPORTS) == set(declared_functions())


def test_every_kernel_unit_is_built():
    # the library is linked from several compilation units (each with its own
    # scheduling options): every HIP source beside ds_topk.hip is one of them,
    # and every launcher ds_topk.hip declares is defined in one
    from sampling_topk_selection_amd import build as b

    csrc = os.path.join(ROOT, "sampling_topk_selection_amd", "csrc")
    units = {os.path.abspath(u if isinstance(u, str) else u[0]) for u in b.UNITS}
    hips = {os.path.abspath(os.path.join(csrc, f)) for f in os.listdir(csrc) if f.endswith(".hip")}
    assert units == hips - {os.path.abspath(b.CALIB_SRC)}
    main = open(b.SRC).read()
    launchers = set(re.findall(r"^hipError_t (ds_topk_launch_\w+)\(", main, flags=re.M))
    assert launchers
    others = "".join(open(u).read() for u in units if u != os.path.abspath(b.SRC))
    for name in launchers:
        assert re.search(r"^hipError_t %s\(.*\{" % name, others, flags=re.M), name
    assert set(b.KERNEL_SOURCES) >= units and set(b.DEPS) >= units


def test_binds_to_one_hip_runtime(pkg):
    maps = open("/proc/self/maps").read()
    libs = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(libs) == 1, libs


def test_status_strings(pkg):
    for st in range(6):
        s = pkg.ds_topk_status_string(st)
        assert s.startswith("DS_")
    assert pkg.ds_topk_status_string(99) == "unknown status"
    assert pkg.ds_topk_version() >= 100


BF, F32 = 0, 1
FAKE = 1 << 20  # never dereferenced: argument errors return first


@pytest.mark.parametrize("args,status", [
    ((BF, 4, 100, 104, 0), 1),        # k < 1
    ((BF, 4, 100, 104, 101), 1),      # k > n
    ((BF, -1, 100, 104, 4), 1),       # batch < 0
    ((BF, 4, 0, 8, 1), 1),            # n < 1
    ((BF, 4, 100, 96, 4), 1),         # row_stride < n
    ((BF, 4, 5000, 5000, 4097), 2),   # k > 4096
    ((7, 4, 100, 104, 4), 2),         # dtype
    ((BF, 4, 1 << 31, 1 << 31, 4), 2),  # n beyond int32
    ((BF, 4, 100, 100, 4), 3),        # bf16 pitch 200 B
    ((F32, 4, 100, 102, 4), 3),       # fp32 pitch 408 B
])
def test_validation_errors(pkg, args, status):
    dtype, batch, n, rs, k = args
    st = pkg.ds_topk(FAKE, dtype, batch, n, rs, k, 0, 0, FAKE, None, None)
    assert st == status, pkg.ds_topk_last_error()
    assert pkg.ds_topk_last_error()
    st2, _ = pkg.ds_topk_plan_for(dtype, batch, n, rs, k)
    assert st2 == status


def test_pointer_errors(pkg):
    assert pkg.ds_topk(None, BF, 4, 64, 64, 8, 0, 0, FAKE, None, None) == 1
    assert pkg.ds_topk(FAKE, BF, 4, 64, 64, 8, 0, 0, None, None, None) == 1
    assert pkg.ds_topk(FAKE, BF, 4, 64, 64, 8, 0, 1, FAKE, None, None) == 1  # values wanted, no buffer
    assert pkg.ds_topk(FAKE + 2, BF, 4, 64, 64, 8, 0, 0, FAKE, None, None) == 3  # misaligned base
    assert pkg.ds_topk_async(FAKE, BF, 4, 64, 64, 8, 0, 0, FAKE, None, None, None) == 1  # no status word
    assert pkg.ds_topk_lengths(FAKE, BF, 4, 64, 64, 8, None, 0, 0, FAKE, None, None) == 1  # no lengths
    assert pkg.ds_topk_lengths(FAKE, BF, 4, 64, 64, 8, FAKE, 3, 0, FAKE, None, None) == 1
    assert pkg.ds_topk_sample(FAKE, BF, 4, 64, 64, 8, None, FAKE, FAKE, FAKE, None) == 1
    assert pkg.ds_topk_sample(FAKE, BF, 4, 64, 64, 8, FAKE, FAKE, FAKE, None, None) == 1
    assert pkg.ds_topk_sample(FAKE, BF, 4, 64, 64, 65, FAKE, FAKE, FAKE, FAKE, None) == 1  # k > n
    assert pkg.ds_topk_sample(FAKE, BF, 4, 8192, 8192, 4097, FAKE, FAKE, FAKE, FAKE, None) == 2  # k > 4096
    for ib in (2, 16):  # index_bytes neither 4 nor 8
        assert pkg.ds_topk_ex(FAKE, BF, 4, 64, 64, 8, 0, 0, FAKE, None, ib) == 1
    for order in (-1, 3):  # not a ds_topk_order
        assert pkg.ds_topk(FAKE, BF, 4, 64, 64, 8, order, 0, FAKE, None, None) == 1
        assert pkg.ds_topk_plan_for(BF, 4, 64, 64, 8, order)[0] == 1
    for order in (pkg.DS_ORDER_NONE, pkg.DS_ORDER_INDEX, pkg.DS_ORDER_VALUE):
        assert pkg.ds_topk_plan_for(BF, 4, 64, 64, 8, order)[0] == 0


def test_noalloc_host_checks(pkg):
    """The no-alloc entry point checks its arguments like ds_topk_async, and
    rejects a row whose split-row state exceeds its static array, all before
    any HIP call."""
    na = pkg.ds_topk_async_noalloc
    assert na(FAKE, BF, 4, 64, 64, 8, 0, 0, FAKE, None, None, None) == 1  # no status word
    assert na(None, BF, 4, 64, 64, 8, 0, 0, FAKE, None, FAKE, None) == 1
    assert na(FAKE, BF, 4, 64, 64, 65, 0, 0, FAKE, None, FAKE, None) == 1  # k > n
    assert na(FAKE + 2, BF, 4, 64, 64, 8, 0, 0, FAKE, None, FAKE, None) == 3
    assert na(FAKE, BF, 0, 64, 64, 8, 0, 0, FAKE, None, FAKE, None) == 0  # no rows
    n, k = 1 << 23, 4096  # 256 segments publishing 9216 entries each: about 21 MB for one row
    st, p = pkg.ds_topk_plan_for(BF, 1, n, n, k)
    assert st == 0 and p.segments == 256
    assert p.segments * (32 + 4 * 2048 + 8 * p.publish_capacity) > pkg.DS_TOPK_NOALLOC_SCRATCH_BYTES
    assert na(FAKE, BF, 1, n, n, k, 0, 0, FAKE, None, FAKE, None) == 2
    assert "static scratch" in pkg.ds_topk_last_error()


def test_k_limits_from_pages(pkg):
    import json

    lim = json.load(open(os.path.join(ROOT, "tests", "golden", "page_limits.json")))["k_max"]["value"]
    assert pkg.ds_topk_plan_for(BF, 1, 8192, 8192, lim)[0] == 0
    assert pkg.ds_topk_plan_for(BF, 1, 8192, 8192, lim + 1)[0] == 2


def test_batch_zero_is_noop(pkg):
    # valid arguments, zero rows: returns before any HIP call
    assert pkg.ds_topk(FAKE, BF, 0, 64, 64, 8, 0, 0, FAKE, None, None) == 0


@pytest.mark.parametrize("cfg", ["C1", "C2", "C3", "C4", "C5"])
def test_plans_for_workloads(pkg, cfg):
    from workloads import CONFIGS

    c = CONFIGS[cfg]
    dt = BF if c["dtype"] == "bf16" else F32
    st, p = pkg.ds_topk_plan_for(dt, c["batch"], c["n"], c["n"], c["k"], int(c["sorted_index"]),
                                 int(c["return_value"]))
    assert st == 0
    epv = 8 if dt == BF else 4
    n_vec = -(-c["n"] // epv)
    assert 1 <= p.segments <= 256
    assert p.segments * p.segment_vectors >= n_vec > (p.segments - 1) * p.segment_vectors
    tile = p.threads * epv  # elements in one tile (one 16-byte vector per thread)
    assert p.tiles_per_chunk >= 1
    assert p.capacity >= 2 * tile  # the two seed tiles fit an empty buffer
    assert p.capacity >= c["k"] + tile  # k kept plus a tile appended
    assert p.grid == c["batch"] * p.segments
    if p.segments > 1:
        assert p.workspace_bytes >= c["batch"] * p.segments * c["k"] * 8


def test_forced_segments(pkg):
    try:
        pkg.ds_topk_set_overrides(7, 0)
        st, p = pkg.ds_topk_plan_for(BF, 4, 204800, 204800, 1024)
        assert st == 0 and p.segments == 7
        pkg.ds_topk_set_overrides(100000, 0)
        st, p = pkg.ds_topk_plan_for(BF, 4, 64, 64, 8)
        assert st == 0 and p.segments == 8  # at most one segment per 16-byte vector
    finally:
        pkg.ds_topk_set_overrides(0, 0)
