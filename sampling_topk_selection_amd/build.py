"""Builds libds_topk.so in-tree with hipcc for gfx950.

    python -m sampling_topk_selection_amd.build
"""

from __future__ import annotations

import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "ds_topk.hip")
# the selection with its sampling step, compiled as a unit of its own
SAMPLE_SRC = os.path.join(HERE, "csrc", "sample_fused.hip")
# the 16384-entry instances, a unit of their own with their own scheduling option
BIGK_SRC = os.path.join(HERE, "csrc", "bigk.hip")
BIGK_FLAGS = ("-mllvm", "-amdgpu-use-amdgpu-trackers")
# the bf16 8192-entry instance, likewise
BF16_SRC = os.path.join(HERE, "csrc", "rows_bf16.hip")
BF16_FLAGS = ("-mllvm", "-structurizecfg-skip-uniform-regions")
DEPS = [SRC, SAMPLE_SRC, BIGK_SRC, BF16_SRC, os.path.join(HERE, "csrc", "topk_kernels.hpp"), os.path.join(HERE, "csrc", "sample_kernels.hpp"),
        os.path.join(ROOT, "include", "ds_topk.h")]
# the library's compilation units, with the flags each adds
UNITS = [SRC, SAMPLE_SRC, (BIGK_SRC, BIGK_FLAGS), (BF16_SRC, BF16_FLAGS)]
LIB = os.path.join(HERE, "libds_topk.so")
# Measurement build of the same sources: the kernels also note phase
# timestamps (DSTK_TIMING); read by sampling_topk_selection_amd.phases.
TIMING_LIB = os.path.join(HERE, "libds_topk_timing.so")
CALIB_SRC = os.path.join(HERE, "csrc", "calib.hip")
CALIB_LIB = os.path.join(HERE, "libds_calib.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Files whose content decides the top-k kernels' code (for tagging profiles).
KERNEL_SOURCES = (SRC, SAMPLE_SRC, BIGK_SRC, BF16_SRC, os.path.join(HERE, "csrc", "topk_kernels.hpp"),
                  os.path.join(ROOT, "include", "ds_topk.h"), os.path.abspath(__file__))


def kernel_source_sha() -> str:
    """Short hash of the kernel sources and build flags: a counter summary
    taken on other sources no longer describes the kernel."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-mcode-object-version=5",
    # keep the compiler from emitting packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the kernels issue LDS atomics from one lane with a wave-uniform amount;
    # the atomic optimizer would wrap each in a scan over the active lanes
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    # the tail steps are chains of short dependent LDS and cross-lane steps
    # inside one workgroup; the ILP-first machine scheduler overlaps more of
    # them than the default occupancy-first one (measured on back-to-back
    # launches: fp32 64 x 129280 k=512 -0.4 us, bf16 4 x 204800 k=1024 -0.3 us)
    "-mllvm", "-amdgpu-sched-strategy=max-ilp",
    "-Wall",
]


def stale(lib: str = LIB, deps=None) -> bool:
    deps = DEPS if deps is None else deps
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    return any(os.path.getmtime(d) > t for d in deps)


def _run(cmd, verbose: bool) -> None:
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)


def _hipcc(src, lib: str, verbose: bool, extra=()) -> None:
    """Compile and link `src` (a path, or a list of paths and (path, flags)
    pairs whose flags apply to that unit only) into the shared library `lib`."""
    tmp = lib + ".tmp%d" % os.getpid()
    srcs = [src] if isinstance(src, str) else list(src)
    units = [(s, ()) if isinstance(s, str) else (s[0], tuple(s[1])) for s in srcs]
    base = [HIPCC] + FLAGS + list(extra) + ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    if all(not f for _, f in units):
        _run(base + ["-o", tmp] + [s for s, _ in units], verbose)
    else:
        # one object per unit (each with its own device code), then one link
        objs = []
        try:
            for i, (s, f) in enumerate(units):
                o = "%s.%d.o" % (tmp, i)
                _run([a for a in base if a != "-shared"] + list(f) + ["-c", "-o", o, s], verbose)
                objs.append(o)
            _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
        finally:
            for o in objs:
                if os.path.exists(o):
                    os.remove(o)
    os.replace(tmp, lib)


def build(force: bool = True, verbose: bool = False, timing: bool = True) -> str:
    """Build libds_topk.so (the library), libds_calib.so (benchmark
    calibration kernels) and, with `timing`, libds_topk_timing.so (the
    library with phase timestamps, for measurement only)."""
    if force or stale():
        _hipcc(UNITS, LIB, verbose)
    if force or stale(CALIB_LIB, [CALIB_SRC]):
        _hipcc(CALIB_SRC, CALIB_LIB, verbose)
    if timing and (force or stale(TIMING_LIB)):
        _hipcc(UNITS, TIMING_LIB, verbose, ["-DDSTK_TIMING"])
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose=True))
    sys.exit(0)
