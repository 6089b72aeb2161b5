"""Summaries of rocprofv3 output for the committed profiles.

    python -m sampling_topk_selection_amd.profiling stats <kernel_stats.csv> <out.txt> "<command>"
    python -m sampling_topk_selection_amd.profiling traffic <fetch_counter_collection.csv> \
        <write_counter_collection.csv> <out.txt> <kernel-substring> <copy-bytes> "<commands>"

`stats` turns a `--kernel-trace --stats -f csv` kernel table into a short
text table (calls, average / min / max duration per kernel).

`traffic` reads two `--pmc` runs (FETCH_SIZE, then WRITE_SIZE; both in KiB
per dispatch) of a program that launched the top-k kernel and the plain copy
kernel of the calibration library on `copy-bytes` bytes.  The copy reads and
writes exactly `copy-bytes`, which gives one scale factor per counter; the
top-k kernel's average counter times that factor is its HBM traffic per
launch.  The summary records the kernel-source hash so that a later build
of different kernels does not reuse it.
"""

from __future__ import annotations

import csv
import sys
from collections import defaultdict

from .build import kernel_source_sha

COPY_KERNEL = "k_copy"


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def stats(stats_csv: str, out_txt: str, command: str) -> None:
    rows = _rows(stats_csv)
    total = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
    lines = ["# rocprofv3 kernel statistics", "# command: %s" % command,
             "# kernel_source_sha: %s" % kernel_source_sha(), "",
             "%-70s %7s %11s %11s %11s %7s" % ("kernel", "calls", "avg_us", "min_us", "max_us", "time%")]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append("%-70s %7d %11.3f %11.3f %11.3f %7.2f" % (
            r["Name"][:70], int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, 100.0 * float(r["TotalDurationNs"]) / total))
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")


def _counter_means(path: str, counter: str):
    acc = defaultdict(list)
    for r in _rows(path):
        if r.get("Counter_Name") != counter:
            continue
        acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}


def _pick(means, sub):
    hits = [k for k in means if sub in k]
    if len(hits) != 1:
        raise SystemExit("expected one kernel matching %r, found %s" % (sub, hits))
    return hits[0]


def traffic(fetch_csv: str, write_csv: str, out_txt: str, kernel_sub: str, copy_bytes: int, commands: str) -> None:
    fm, fn = _counter_means(fetch_csv, "FETCH_SIZE")
    wm, wn = _counter_means(write_csv, "WRITE_SIZE")
    kf, kw = _pick(fm, kernel_sub), _pick(wm, kernel_sub)
    cf, cw = _pick(fm, COPY_KERNEL), _pick(wm, COPY_KERNEL)
    fetch_scale = copy_bytes / (fm[cf] * 1024.0)
    write_scale = copy_bytes / (wm[cw] * 1024.0)
    fetch_b = round(fm[kf] * 1024.0 * fetch_scale)
    write_b = round(wm[kw] * 1024.0 * write_scale)
    lines = [
        "# HBM traffic per launch from rocprofv3 counters, scaled by a copy of known size",
        "# commands: %s" % commands,
        "kernel: %s" % kf,
        "kernel_source_sha: %s" % kernel_source_sha(),
        "dispatches_fetch: %d" % fn[kf],
        "dispatches_write: %d" % wn[kw],
        "FETCH_SIZE_KiB_per_dispatch: %.1f" % fm[kf],
        "WRITE_SIZE_KiB_per_dispatch: %.1f" % wm[kw],
        "copy_bytes: %d" % copy_bytes,
        "copy_FETCH_SIZE_KiB: %.1f" % fm[cf],
        "copy_WRITE_SIZE_KiB: %.1f" % wm[cw],
        "fetch_scale: %.4f" % fetch_scale,
        "write_scale: %.4f" % write_scale,
        "fetch_bytes_per_launch: %d" % fetch_b,
        "write_bytes_per_launch: %d" % write_b,
        "hbm_bytes_per_launch: %d" % (fetch_b + write_b),
    ]
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    a = sys.argv[1:]
    if a and a[0] == "stats" and len(a) == 4:
        stats(a[1], a[2], a[3])
    elif a and a[0] == "traffic" and len(a) == 7:
        traffic(a[1], a[2], a[3], a[4], int(a[5]), a[6])
    else:
        raise SystemExit(__doc__)
