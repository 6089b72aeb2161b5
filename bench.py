#!/usr/bin/env python3
"""Benchmark of row-wise small-k top-k on one MI355X.

Metric (the pages' only one: effective memory bandwidth, since top-k does no
floating-point math -- aiutil project card "deepseek-ai/DeepSelect",
关键技术亮点 item 4): algorithmic bytes / time, where algorithmic bytes per
row = n * element size (every valid input element read once) + 4k (int32
indices) + k * element size when values are returned.

One step = one top-k call on each of the two shapes the metric names, back
to back on one stream:
  * Lightning-Indexer shape: bf16 4 x 204800, k = 1024, unsorted, indices only
    (CSDN page "DeepSeek 一次开源三个仓库", section 三 usage example);
  * sampler shape: fp32 64 x 129280, k = 512, sorted indices, values
    (same page and section, the fp32 sampling performance group).
Inputs are seeded synthetic rows already resident in HBM.  Each call reads
a different copy of its input (the copies span >= 1 GB), so every call
streams from HBM rather than from the 256 MB last-level cache.

Timing uses HIP events on the stream the kernels run on.  Each call is the
enqueue-only entry point (ds_topk_async) with its own device status word;
the statuses are read after the timed region and must all be DS_OK.  The
synchronous entry point's per-call latency (kernel + status readback) is
reported beside it.

Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective HBM GB/s (% peak), bf16 4×204800 k=1024 & fp32 64×129280 k=512"
PEAK_GBS = 8000.0  # MI355X HBM3E
STEP_WORKLOADS = ("C2", "C3")
DOMINANT = "C3"
TRAFFIC_FILES = {"C2": "topk_rows_bf16_indexer_4x204800_k1024_traffic.txt",
                 "C3": "topk_rows_fp32_sampler_64x129280_k512_traffic.txt"}
STATS_FILE = "topk_rows_bench_step_indexer_bf16_4x204800_sampler_fp32_64x129280_kernel_stats.txt"
KERNEL_NAMES = {"C2": "topk_rows<2, 512, 2, 8192>", "C3": "topk_rows<4, 512, 4, 8192>"}


def _current(path: str):
    """The lines of a committed profile summary, if it was taken on the
    current kernel sources; else None."""
    if not os.path.exists(path):
        return None
    from sampling_topk_selection_amd.build import kernel_source_sha

    lines = open(path).read().splitlines()
    if not any(l.replace("#", "").strip() == "kernel_source_sha: %s" % kernel_source_sha() for l in lines):
        return None
    return lines


def load_traffic(workload: str):
    """HBM bytes per launch (fetch, write, total) from the committed
    rocprofv3 counter summary, if it was taken on the current kernel
    sources; else None."""
    lines = _current(os.path.join(ROOT, "profiles", TRAFFIC_FILES[workload]))
    if lines is None:
        return None
    kv = {}
    for line in lines:
        if ":" in line and not line.startswith("#"):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    try:
        return {k: int(float(kv[k + "_bytes_per_launch"])) for k in ("fetch", "write", "hbm")}
    except (KeyError, ValueError):
        return None


def load_profiled_avg_us(workload: str):
    """The kernel's average duration in the committed rocprofv3 kernel
    statistics of the bench command, if taken on the current sources."""
    lines = _current(os.path.join(ROOT, "profiles", STATS_FILE))
    if lines is None:
        return None
    for line in lines:
        if KERNEL_NAMES[workload] in line:
            # name, calls, avg_us, min_us, max_us, time%
            return float(line.split(")")[-1].split()[1])
    return None


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate-gb", type=float, default=1.0,
                    help="total size of the rotated input copies per workload (0 = one buffer, warm)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle CPU-baseline budget")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed steps (for profiler runs)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run the copy calibration kernel (for counter scaling)")
    return ap.parse_args()


def main() -> int:
    args = parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(rows are independent; see the design notes). Use --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from sampling_topk_selection_amd import build as builder

    if not os.path.exists(builder.LIB) or not os.path.exists(builder.CALIB_LIB):
        builder.build(force=False)
    import ctypes

    import sampling_topk_selection_amd as pkg
    from workloads import make_workload

    pkg.load_library()
    calib = ctypes.CDLL(builder.CALIB_LIB)
    calib.calib_empty.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    calib.calib_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                 ctypes.c_void_p]
    calib.calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_void_p]

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    # ---------------------------------------------------------------- inputs
    W = {}
    for cfg in STEP_WORKLOADS:
        w = make_workload(cfg)
        raw = np.ascontiguousarray(w.raw)
        x0 = (torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16) if w.dtype == "bf16"
              else torch.from_numpy(raw)).to(dev)
        copies = max(1, int(math.ceil(args.rotate_gb * 1e9 / x0.numel() / x0.element_size())))
        X = torch.empty((copies,) + tuple(x0.shape), dtype=x0.dtype, device=dev)
        X.copy_(x0.unsqueeze(0).expand_as(X))
        dt = pkg.DS_DTYPE_BF16 if w.dtype == "bf16" else pkg.DS_DTYPE_F32
        idx = torch.empty((w.batch, w.k), dtype=torch.int32, device=dev)
        val = torch.empty((w.batch, w.k), dtype=x0.dtype, device=dev) if w.return_value else None
        st, plan = pkg.ds_topk_plan_for(dt, w.batch, w.n, w.row_stride, w.k, int(w.sorted_index),
                                        int(w.return_value))
        assert st == 0
        W[cfg] = dict(w=w, X=X, copies=copies, dt=dt, idx=idx, val=val, plan=plan,
                      bytes=w.algorithmic_bytes(), x0=x0)

    nstatus = args.warmup + 2 * args.steps + 4 * max(20, args.steps) + 64
    status = torch.zeros(nstatus, dtype=torch.int32, device=dev)
    slot = [0]

    def call(cfg, copy_i):
        d = W[cfg]
        w = d["w"]
        x = d["X"][copy_i % d["copies"]]
        s = status[slot[0] % nstatus:]
        slot[0] += 1
        rc = pkg.ds_topk_async(x.data_ptr(), d["dt"], w.batch, w.n, w.row_stride, w.k,
                               int(w.sorted_index), int(w.return_value), d["idx"].data_ptr(),
                               d["val"].data_ptr() if d["val"] is not None else None, s.data_ptr(), sptr)
        if rc != 0:
            raise RuntimeError("ds_topk_async failed: %s" % pkg.ds_topk_last_error())

    def step(i):
        for cfg in STEP_WORKLOADS:
            call(cfg, i)

    # ---------------------------------------------------------------- warmup + timed steps
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / args.steps
    step_bytes = sum(W[c]["bytes"] for c in STEP_WORKLOADS)
    value = step_bytes / (step_ms * 1e-3) / 1e9

    per = {}

    def per_call_ms(fn, reps):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            fn(i)
            b.record(stream)
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in evs)
        return sum(ts) / len(ts), ts[len(ts) // 2], ts[len(ts) // 10], ts[(9 * len(ts)) // 10]

    reps = max(20, args.steps)
    for cfg in STEP_WORKLOADS:
        # ------------------------------------------------------------ calibration (also in profiler runs)
        d = W[cfg]
        w = d["w"]
        grid = d["plan"].grid
        out_buf = torch.empty(max(1, grid), dtype=torch.int32, device=dev)
        nbytes_in = w.batch * w.row_stride * w.elem_size

        def rd(i, c=cfg, g=grid, ob=out_buf, nb=nbytes_in):
            X = W[c]["X"]
            calib.calib_read(X[i % W[c]["copies"]].data_ptr(), nb, g, ob.data_ptr(), sptr)

        ravg, rmed, _, _ = per_call_ms(rd, reps)
        # launch floor: empty kernels of the same grid, back to back
        calib.calib_empty(grid, 20, sptr)
        fa, fb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fa.record(stream)
        calib.calib_empty(grid, 200, sptr)
        fb.record(stream)
        torch.cuda.synchronize()
        empty_us = fa.elapsed_time(fb) * 1e3 / 200
        per[cfg] = {
            "shape": "%s %dx%d k=%d sorted=%d values=%d" % (w.dtype, w.batch, w.n, w.k, w.sorted_index,
                                                            w.return_value),
            "algorithmic_bytes": d["bytes"],
            "segments_per_row": d["plan"].segments,
            "workgroups": grid,
            "input_copies": d["copies"],
            "calib_stream_read_us": round(ravg * 1e3, 3),
            "calib_stream_read_GBps": round(nbytes_in / (ravg * 1e-3) / 1e9, 1),
            "calib_empty_kernel_us": round(empty_us, 3),
            "hbm_traffic_bytes_per_launch": load_traffic(cfg),
        }
        if args.no_extras:
            continue
        # ------------------------------------------------------------ per-call kernel time
        avg, med, p10, p90 = per_call_ms(lambda i, c=cfg: call(c, i), reps)
        wavg, wmed, _, _ = per_call_ms(lambda i, c=cfg: call(c, 0), reps)
        per[cfg].update({
            "us_per_call_mean": round(avg * 1e3, 3),
            "us_per_call_median": round(med * 1e3, 3),
            "us_p10": round(p10 * 1e3, 3),
            "us_p90": round(p90 * 1e3, 3),
            "GBps": round(d["bytes"] / (avg * 1e-3) / 1e9, 1),
            "pct_peak": round(100.0 * d["bytes"] / (avg * 1e-3) / 1e9 / PEAK_GBS, 2),
            "rows_per_s": round(w.batch / (avg * 1e-3), 1),
            "warm_us_per_call": round(wavg * 1e3, 3),
            "warm_GBps": round(d["bytes"] / (wavg * 1e-3) / 1e9, 1),
            "pct_of_stream_read": round(100.0 * ravg / avg, 1),
        })

    if not args.no_extras:
        # synchronous entry point (kernel + stream wait + status check) per
        # call: through the C ABI on preallocated outputs, and through the
        # Python topk(), which also allocates its outputs
        for cfg in STEP_WORKLOADS:
            d = W[cfg]
            w = d["w"]
            x = d["x0"]

            def sync_call(c=cfg, xx=x):
                dd = W[c]
                ww = dd["w"]
                rc = pkg.ds_topk(xx.data_ptr(), dd["dt"], ww.batch, ww.n, ww.row_stride, ww.k,
                                 int(ww.sorted_index), int(ww.return_value), dd["idx"].data_ptr(),
                                 dd["val"].data_ptr() if dd["val"] is not None else None, sptr)
                if rc != 0:
                    raise RuntimeError("ds_topk failed: %s" % pkg.ds_topk_last_error())

            r = 50
            for _ in range(3):
                sync_call()
            t = time.perf_counter()
            for _ in range(r):
                sync_call()
            per[cfg]["sync_call_us"] = round((time.perf_counter() - t) / r * 1e6, 1)
            for _ in range(3):
                pkg.topk(x, w.k, sorted_index=w.sorted_index, return_value=w.return_value)
            t = time.perf_counter()
            for _ in range(r):
                pkg.topk(x, w.k, sorted_index=w.sorted_index, return_value=w.return_value)
            per[cfg]["sync_call_python_us"] = round((time.perf_counter() - t) / r * 1e6, 1)
            # the same kernels enqueued back to back on one (warm) input: the
            # kernel time the synchronous call adds its wait to
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            for _ in range(r):
                call(cfg, 0)
            b_.record(stream)
            torch.cuda.synchronize()
            per[cfg]["warm_back_to_back_us"] = round(a_.elapsed_time(b_) * 1e3 / r, 3)

    modes = {}
    if not args.no_extras:
        # the output-order and per-row-length modes, warm, back to back
        def mode_us(x, w, reps=40, **kw):
            st1 = torch.zeros(1, dtype=torch.int32, device=dev)
            for _ in range(3):
                pkg.topk_async(x, w.k, st1, n=w.n, **kw)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                pkg.topk_async(x, w.k, st1, n=w.n, **kw)
            b.record(stream)
            torch.cuda.synchronize()
            assert int(st1.item()) == 0
            return a.elapsed_time(b) * 1e3 / reps

        w3 = W[DOMINANT]["w"]
        x3 = W[DOMINANT]["x0"]
        for name, kw in (("index", dict(sorted_index=True)), ("value", dict(sorted_value=True)),
                         ("none", dict()), ("index_int64", dict(sorted_index=True, indices_type=torch.int64))):
            modes["C3_order_%s_us" % name] = round(mode_us(x3, w3, return_value=True, **kw), 3)
        w4 = make_workload("C4")
        x4 = torch.from_numpy(np.ascontiguousarray(w4.raw).view(np.int16)).view(torch.bfloat16).to(dev)
        l4 = torch.tensor(w4.meta["lengths"], dtype=torch.int32, device=dev)
        modes["C4_neg_inf_tails_us"] = round(mode_us(x4, w4, return_value=True), 3)
        modes["C4_lengths_us"] = round(mode_us(x4, w4, return_value=True, lengths=l4), 3)
        modes["C4_valid_bytes"] = int(sum(w4.meta["lengths"]) * 2 + w4.batch * w4.k * 6)
        # heavy ties at the largest k: 16 levels ascending along each row
        w5 = make_workload("C5")
        x5 = torch.from_numpy(np.ascontiguousarray(w5.raw).view(np.int16)).view(torch.bfloat16).to(dev)
        modes["C5_max_k_us"] = round(mode_us(x5, w5, return_value=True, sorted_index=True), 3)
        # many short rows: one wave per row
        for (bsz, nn, kk) in ((4096, 256, 64), (16384, 128, 16)):
            gs = torch.Generator(device="cpu").manual_seed(bsz + nn)
            xs = torch.randn(bsz, nn, generator=gs).to(torch.bfloat16).to(dev)

            class _W:  # the shape mode_us needs
                k, n = kk, nn
            modes["short_rows_bf16_%dx%d_k%d_us" % (bsz, nn, kk)] = round(mode_us(xs, _W, return_value=True), 3)
        # one token per row from the top-k (synchronous calls, with their status readback)
        g = torch.Generator(device="cpu").manual_seed(3)
        tt = (0.5 + 1.5 * torch.rand(w3.batch, generator=g)).to(dev)
        pp = (0.5 + 0.5 * torch.rand(w3.batch, generator=g)).to(dev)
        uu = torch.rand(w3.batch, generator=g).to(dev)
        for _ in range(3):
            pkg.sample(x3, w3.k, tt, pp, uu)
        t = time.perf_counter()
        for _ in range(30):
            pkg.sample(x3, w3.k, tt, pp, uu)
        modes["C3_sample_sync_call_us"] = round((time.perf_counter() - t) / 30 * 1e6, 1)

    if args.calib_copy:
        # a plain copy of the sampler input: known traffic for counter scaling
        d = W[DOMINANT]
        src = d["X"][0]
        dst = torch.empty_like(src)
        for _ in range(5):
            calib.calib_copy(src.data_ptr(), dst.data_ptr(), src.numel() * src.element_size(), 2048, sptr)
        torch.cuda.synchronize()

    # the dominant kernel alone, launched back to back: average launch
    # duration over the timed region (events on the stream it runs on)
    dom_reps = max(20, args.steps)
    for i in range(3):
        call(DOMINANT, i)
    a_ev = torch.cuda.Event(enable_timing=True)
    b_ev = torch.cuda.Event(enable_timing=True)
    a_ev.record(stream)
    for i in range(dom_reps):
        call(DOMINANT, i)
    b_ev.record(stream)
    torch.cuda.synchronize()
    dom_us = a_ev.elapsed_time(b_ev) * 1e3 / dom_reps

    torch.cuda.synchronize()
    st = status.cpu().numpy()
    if np.any(st != 0):
        raise RuntimeError("a timed call reported status %s" % np.unique(st).tolist())

    # ---------------------------------------------------------------- roofline (dominant kernel)
    from sampling_topk_selection_amd.build import kernel_source_sha

    achieved = W[DOMINANT]["bytes"] / (dom_us * 1e-6) / 1e9
    tr = load_traffic(DOMINANT)
    traffic = tr["hbm"] if tr else None
    prof_us = load_profiled_avg_us(DOMINANT)
    roofline = {
        "bound": "hbm",
        "kernel": "topk_rows<4, 512, %d, %d> (fp32 sampler shape: 64 x 129280, k=512)" % (
            W[DOMINANT]["plan"].tiles_per_chunk, W[DOMINANT]["plan"].capacity),
        "achieved": round(achieved, 1),
        "peak": PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / PEAK_GBS, 4),
        "traffic": traffic,
        "algorithmic_bytes_per_launch": W[DOMINANT]["bytes"],
        "avg_launch_us": round(dom_us, 3),
        "launches_timed": dom_reps,
        # the same ratio with the committed rocprofv3 average of this kernel
        # (profiles/, kernel statistics of the bench command), when taken on
        # the current sources
        "profiled_avg_us": prof_us,
        "frac_profiled": round(W[DOMINANT]["bytes"] / (prof_us * 1e-6) / 1e9 / PEAK_GBS, 4) if prof_us else None,
        "kernel_source_sha": kernel_source_sha(),
    }

    # ---------------------------------------------------------------- CPU baseline: the oracle
    cpu = None
    if not args.no_cpu:
        import oracle

        oracle.build(force=False)
        threads = oracle.max_threads()
        reps, t_cpu, mism = 0, 0.0, 0
        gpu_out = {}
        for cfg in STEP_WORKLOADS:
            d = W[cfg]
            w = d["w"]
            v, i = pkg.topk(d["x0"], w.k, sorted_index=w.sorted_index, return_value=w.return_value)
            gpu_out[cfg] = (i.cpu().numpy(),
                            None if v is None else (v.cpu().view(torch.int16).numpy().view(np.uint16)
                                                    if w.dtype == "bf16" else v.cpu().numpy()))
        while True:
            for cfg in STEP_WORKLOADS:
                w = W[cfg]["w"]
                t = time.perf_counter()
                s, oi, ov = oracle.topk(w.raw, w.dtype, w.n, w.k, w.sorted_index, w.return_value,
                                        nthreads=0)
                t_cpu += time.perf_counter() - t
                if reps == 0:  # parity of the timed outputs against the oracle
                    gi, gv = gpu_out[cfg]
                    same = (np.array_equal(gi, oi) if w.sorted_index
                            else np.array_equal(np.sort(gi, 1), np.sort(oi, 1)))
                    if gv is not None:
                        same = same and np.array_equal(gv.view(np.uint8), ov.view(np.uint8))
                    mism += 0 if (s == 0 and same) else 1
            reps += 1
            if t_cpu >= args.cpu_seconds:
                break
        cpu = {
            "value": round(step_bytes * reps / t_cpu / 1e9, 3),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": "%d repetitions of the full step (bf16 4x204800 k=1024 + fp32 64x129280 k=512), "
                      "OpenMP over rows (the 4-row shape uses at most 4 threads)" % reps,
            "ms_per_step": round(t_cpu / reps * 1e3, 2),
            "gpu_outputs_match_oracle": mism == 0,
        }

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u64",
        "data": "synthetic",
        "pct_peak": round(100.0 * value / PEAK_GBS, 2),
        "config": {
            "workload": "row-wise top-k: lightning-indexer bf16 4x204800 k=1024 (unsorted, indices only) + "
                        "sampler fp32 64x129280 k=512 (sorted indices, values), one call each per step",
            "input_dtypes": ["bf16", "f32"],
            "compare_keys": "order-preserving u16/u32 value keys + column, as u64",
            "cold_hbm": args.rotate_gb > 0,
            "wall_ms_per_step": round(wall / args.steps * 1e3, 5),
            "per_workload": per,
            "modes": modes,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
