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
DEPS = [SRC, os.path.join(HERE, "csrc", "topk_kernels.hpp"), os.path.join(HERE, "csrc", "sample_kernels.hpp"),
        os.path.join(ROOT, "include", "ds_topk.h")]
LIB = os.path.join(HERE, "libds_topk.so")
CALIB_SRC = os.path.join(HERE, "csrc", "calib.hip")
CALIB_LIB = os.path.join(HERE, "libds_calib.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Files whose content decides the top-k kernels' code (for tagging profiles).
KERNEL_SOURCES = (SRC, os.path.join(HERE, "csrc", "topk_kernels.hpp"), os.path.join(ROOT, "include", "ds_topk.h"),
                  os.path.abspath(__file__))


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
    "-Wall",
]


def stale(lib: str = LIB, deps=None) -> bool:
    deps = DEPS if deps is None else deps
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    return any(os.path.getmtime(d) > t for d in deps)


def _hipcc(src: str, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
                             "-o", tmp, src]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, lib)


def build(force: bool = True, verbose: bool = False) -> str:
    """Build libds_topk.so (the library) and libds_calib.so (benchmark
    calibration kernels)."""
    if force or stale():
        _hipcc(SRC, LIB, verbose)
    if force or stale(CALIB_LIB, [CALIB_SRC]):
        _hipcc(CALIB_SRC, CALIB_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose=True))
    sys.exit(0)
