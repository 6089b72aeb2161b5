"""CPU: the host side of bench.py -- the one-GPU guard and the counter
summary it reports as roofline traffic (used only while it describes the
current kernel sources)."""

import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import pytest  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _summary(path):
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    return kv


MIN_READ = {"C2": 4 * 204800 * 2, "C3": 64 * 129280 * 4}


@pytest.mark.parametrize("cfg", ["C2", "C3"])
def test_traffic_summary_is_consistent(cfg):
    path = os.path.join(ROOT, "profiles", bench.TRAFFIC_FILES[cfg])
    kv = _summary(path)
    fetch, write = int(kv["fetch_bytes_per_launch"]), int(kv["write_bytes_per_launch"])
    assert fetch + write == int(kv["hbm_bytes_per_launch"])
    # the copy reads and writes copy_bytes: the scale factors map the counters to bytes
    copy = int(kv["copy_bytes"])
    assert abs(float(kv["fetch_scale"]) * float(kv["copy_FETCH_SIZE_KiB"]) * 1024 - copy) < 0.01 * copy
    assert abs(float(kv["write_scale"]) * float(kv["copy_WRITE_SIZE_KiB"]) * 1024 - copy) < 0.01 * copy
    # at least the algorithmic input bytes are read
    assert fetch >= MIN_READ[cfg]
    assert bench.KERNEL_NAMES[cfg] in kv["kernel"]


def test_traffic_used_only_for_the_current_sources(tmp_path, monkeypatch):
    from sampling_topk_selection_amd.build import kernel_source_sha

    src = os.path.join(ROOT, "profiles", bench.TRAFFIC_FILES["C3"])
    os.makedirs(tmp_path / "profiles")
    dst = tmp_path / "profiles" / bench.TRAFFIC_FILES["C3"]
    shutil.copy(src, dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    current = _summary(src).get("kernel_source_sha") == kernel_source_sha()
    got = bench.load_traffic("C3")
    assert (got["hbm"] == int(_summary(src)["hbm_bytes_per_launch"])) if current else got is None
    text = open(dst).read().replace("kernel_source_sha: ", "kernel_source_sha: x")
    open(dst, "w").write(text)
    assert bench.load_traffic("C3") is None
    os.remove(dst)
    assert bench.load_traffic("C3") is None


def test_profiled_average_read_from_the_kernel_statistics(tmp_path, monkeypatch):
    from sampling_topk_selection_amd.build import kernel_source_sha

    os.makedirs(tmp_path / "profiles")
    dst = tmp_path / "profiles" / bench.STATS_FILE
    rows = ["# rocprofv3 kernel statistics", "# command: x", "# kernel_source_sha: %s" % kernel_source_sha(), "",
            "%-70s %7s %11s %11s %11s %7s" % ("kernel", "calls", "avg_us", "min_us", "max_us", "time%"),
            "%-70s %7d %11.3f %11.3f %11.3f %7.2f" % ("void dstk::topk_rows<4, 512, 4, 8192>(dstk::Params)", 48,
                                                      21.5, 20.0, 30.0, 55.0),
            "%-70s %7d %11.3f %11.3f %11.3f %7.2f" % ("void dstk::topk_rows<2, 512, 2, 8192>(dstk::Params)", 25,
                                                      12.25, 11.0, 14.0, 20.0)]
    open(dst, "w").write("\n".join(rows) + "\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.load_profiled_avg_us("C3") == 21.5
    assert bench.load_profiled_avg_us("C2") == 12.25
    open(dst, "w").write("\n".join(rows).replace("kernel_source_sha: ", "kernel_source_sha: x") + "\n")
    assert bench.load_profiled_avg_us("C3") is None
