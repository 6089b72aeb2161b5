"""CPU: the oracle (oracle/oracle.c) and the host half of the library
(argument checks, planning, the no-alloc size check; the host code of
ds_topk.hip and the units beside it) built with AddressSanitizer and UndefinedBehaviorSanitizer and driven
through their entry points by small C/C++ drivers, which also check the
results they can check without a GPU.  Any sanitizer report fails the run
(-fno-sanitize-recover).  The device code of ds_topk.hip is compiled as usual
(the sanitizers apply to the host side only) and never runs here."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(exe, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.check_call(["gcc", "-std=c11", "-g", "-O1", "-fopenmp"] + SAN +
                          [os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "asan_oracle_driver.c"),
                           "-lm", "-o", exe])
    out = _run(exe, {"OMP_NUM_THREADS": "2"})
    assert "all checks passed" in out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_library_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_driver")
    host_san = []
    for flag in SAN:  # host compilation only
        host_san += ["-Xarch_host", flag]
    cmd = ([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + host_san +
           ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "sampling_topk_selection_amd", "csrc"),
            os.path.join(ROOT, "sampling_topk_selection_amd", "csrc", "ds_topk.hip"),
            os.path.join(ROOT, "sampling_topk_selection_amd", "csrc", "sample_fused.hip"),
            os.path.join(ROOT, "sampling_topk_selection_amd", "csrc", "bigk.hip"),
            os.path.join(ROOT, "sampling_topk_selection_amd", "csrc", "rows_bf16.hip"),
            os.path.join(HERE, "asan_host_driver.cpp"), "-o", exe])
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    # the HIP runtime's own allocations at load are not the library's: no leak check
    out = _run(exe, {"ASAN_OPTIONS": "detect_leaks=0"})
    assert "all checks passed" in out
