"""Phase timing of the top-k kernel (measurement only).

    python -m sampling_topk_selection_amd.phases C3 [--segs S] [--flags F] [--reps R]

Runs a seeded workload through libds_topk_timing.so -- the same sources as
libds_topk.so built with DSTK_TIMING, whose kernels note the constant
100 MHz clock (s_memrealtime, 10 ns ticks) at named points -- and prints,
per phase, the mean time a workgroup spends between the previous noted point
and that one, for the row segments and, on split rows, for the merging
workgroups separately; plus the mean launch span (first start to last end)
and the critical path of the last merge.  The product library is not
touched; this module is not imported by it.
"""

from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TICK_NS = 10.0  # s_memrealtime: 100 MHz
SLOTS = 16
PHASES = ["start", "seed", "scan", "sync", "locate", "(unused)", "publish", "ticket", "metadata", "row_bin",
          "list_load", "refine", "emit"]
PH = {name: i for i, name in enumerate(PHASES)}
CLK_START, CLK_END = 13, 14  # shader clock counter at entry and at the flush


def _load(builder):
    import sampling_topk_selection_amd as pkg

    if not os.path.exists(builder.TIMING_LIB):
        raise ImportError("libds_topk_timing.so not built; run python -m sampling_topk_selection_amd.build")
    lib = pkg.load_library(builder.TIMING_LIB)
    lib.ds_topk_timing_buffer.restype = None
    lib.ds_topk_timing_buffer.argtypes = [ctypes.c_void_p]
    return lib


def summarize(ts: np.ndarray) -> dict:
    """ts: [grid, SLOTS] int64 timestamps of one launch (0 = not noted)."""
    used = ts[:, PH["start"]] != 0
    ts = ts[used]
    clk = ts[:, CLK_START:CLK_END + 1].astype(np.float64)
    ts = ts[:, :len(PHASES)]
    t0 = ts[:, PH["start"]].min()
    ends = ts.max(axis=1)
    # mean shader clock over each workgroup's life: shader clock ticks over
    # constant-clock ticks, from entry to the last note
    ok = (clk[:, 1] > clk[:, 0]) & (ends > ts[:, PH["start"]])
    mhz = (clk[ok, 1] - clk[ok, 0]) / ((ends[ok] - ts[ok, PH["start"]]) * TICK_NS * 1e-3)
    merger = ts[:, PH["metadata"]] != 0
    out = {"workgroups": int(ts.shape[0]), "span_us": float((ends.max() - t0) * TICK_NS / 1e3),
           "clock_mhz": float(np.mean(mhz)) if ok.any() else 0.0,
           "mergers": int(merger.sum())}

    def deltas(rows):
        res = {}
        for r in rows:
            prev = r[PH["start"]]
            for i in range(1, len(PHASES)):
                if r[i]:
                    res.setdefault(PHASES[i], []).append((r[i] - prev) * TICK_NS / 1e3)
                    prev = r[i]
        return {k: float(np.mean(v)) for k, v in res.items()}

    out["segment_us"] = deltas(ts[~merger] if (~merger).any() else ts)
    # the workgroup that ended last (its own phases, from its start)
    slow = ts[np.argmax(ends)]
    out["slowest_us"] = deltas(slow[None, :])
    out["slowest_us"]["start_offset"] = float((slow[PH["start"]] - t0) * TICK_NS / 1e3)
    if merger.any():
        out["merger_us"] = deltas(ts[merger])
        last = ts[merger][np.argmax(ends[merger])]
        path = {"kernel_start_to_merger_start": (last[PH["start"]] - t0)}
        prev = last[PH["start"]]
        for i in range(1, len(PHASES)):
            if last[i]:
                path[PHASES[i]] = last[i] - prev
                prev = last[i]
        out["last_merge_path_us"] = {k: float(v * TICK_NS / 1e3) for k, v in path.items()}
    return out


def run(cfg: str, segs: int = 0, flags: int = 0, reps: int = 10, batch=None):
    import torch

    import sampling_topk_selection_amd as pkg
    from sampling_topk_selection_amd import build as builder
    from workloads import make_workload

    lib = _load(builder)
    w = make_workload(cfg) if batch is None else make_workload(cfg, batch=batch)
    dev = torch.device("cuda:0")
    raw = np.ascontiguousarray(w.raw)
    x = (torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16) if w.dtype == "bf16"
         else torch.from_numpy(raw)).to(dev)
    dt = pkg.DS_DTYPE_BF16 if w.dtype == "bf16" else pkg.DS_DTYPE_F32
    lib.ds_topk_set_overrides(segs, 0, flags)
    plan = pkg.ds_topk_plan()
    st = lib.ds_topk_plan_for(dt, w.batch, w.n, w.row_stride, w.k, int(w.sorted_index), int(w.return_value),
                              ctypes.byref(plan))
    assert st == 0
    grid = max(1, plan.grid)
    buf = torch.zeros((grid, SLOTS), dtype=torch.int64, device=dev)
    idx = torch.empty((w.batch, w.k), dtype=torch.int32, device=dev)
    val = torch.empty((w.batch, w.k), dtype=x.dtype, device=dev) if w.return_value else None
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    res = []
    try:
        for rep in range(reps + 1):
            buf.zero_()
            torch.cuda.synchronize()
            lib.ds_topk_timing_buffer(buf.data_ptr())
            rc = lib.ds_topk_async(x.data_ptr(), dt, w.batch, w.n, w.row_stride, w.k, int(w.sorted_index),
                                   int(w.return_value), idx.data_ptr(), val.data_ptr() if val is not None else None,
                                   status.data_ptr(), stream)
            torch.cuda.synchronize()
            lib.ds_topk_timing_buffer(None)
            assert rc == 0 and int(status.item()) == 0
            if rep:
                res.append(summarize(buf.cpu().numpy()))
    finally:
        lib.ds_topk_timing_buffer(None)
        lib.ds_topk_set_overrides(0, 0, 0)

    def avg(key):
        ks = set().union(*(r.get(key, {}).keys() for r in res))
        return {k: round(float(np.mean([r[key][k] for r in res if k in r.get(key, {})])), 3) for k in ks}

    return {"workload": cfg, "shape": "%s %dx%d k=%d sorted=%d values=%d" % (w.dtype, w.batch, w.n, w.k,
                                                                             w.sorted_index, w.return_value),
            "segments": plan.segments, "grid": plan.grid, "reps": reps,
            "span_us": round(float(np.mean([r["span_us"] for r in res])), 3),
            "clock_mhz": round(float(np.mean([r["clock_mhz"] for r in res])), 1),
            "segment_us": avg("segment_us"), "merger_us": avg("merger_us"), "slowest_us": avg("slowest_us"),
            "last_merge_path_us": avg("last_merge_path_us")}


def format_table(r: dict) -> str:
    lines = ["workload %s (%s): segments %d, grid %d, %d launches" % (
        r["workload"], r["shape"], r["segments"], r["grid"], r["reps"]),
        "mean launch span (first start to last end): %.2f us; mean shader clock %.0f MHz" % (
            r["span_us"], r["clock_mhz"]),
        "%-14s %12s %12s %16s %14s" % ("phase", "segment us", "merger us", "last merge path", "slowest wg")]
    for name in PHASES[1:]:
        s, m, p = r["segment_us"].get(name), r["merger_us"].get(name), r["last_merge_path_us"].get(name)
        w = r["slowest_us"].get(name)
        if s is None and m is None and p is None and w is None:
            continue
        f = lambda v: "%.3f" % v if v is not None else "-"
        lines.append("%-14s %12s %12s %16s %14s" % (name, f(s), f(m), f(p), f(w)))
    lines.append("slowest workgroup started %.3f us after the first" % r["slowest_us"].get("start_offset", 0.0))
    if "kernel_start_to_merger_start" in r["last_merge_path_us"]:
        lines.append("last merger started %.3f us after the first workgroup" %
                     r["last_merge_path_us"]["kernel_start_to_merger_start"])
    return "\n".join(lines)


def main() -> int:
    ap = argparse.ArgumentParser(description="phase timing of the top-k kernel (measurement build)")
    ap.add_argument("workloads", nargs="+")
    ap.add_argument("--segs", type=int, default=0)
    ap.add_argument("--flags", type=int, default=0)
    ap.add_argument("--reps", type=int, default=10)
    args = ap.parse_args()
    for cfg in args.workloads:
        print(format_table(run(cfg, args.segs, args.flags, args.reps)), flush=True)
        print(flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
