"""Build libspecverify.so (HIP, gfx950) in-tree.

    python -m rejection_sampling_verify_12_amd.build
    python -m rejection_sampling_verify_12_amd.build --timeline   (the measurement build)
    python -m rejection_sampling_verify_12_amd.build --checks     (the checks build)

Every HIP source is compiled with packed-FP32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops); the host pass warns that
it does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspecverify.so")
# A measurement build: the same library with SV_TIMELINE=1, whose single
# kernel records every block's start, end, item and CU (bench.py --timeline).
TIMELINE_LIB = os.path.join(PKG, "libspecverify_timeline.so")
# The checks build: the same library with SV_CHECKS=1, whose kernels test
# every index they form against its array's size and record a failure in the
# workspace's second word instead of trapping (tests/test_gpu_checks.py).
CHECKS_LIB = os.path.join(PKG, "libspecverify_checks.so")
SOURCES = ["verify.hip", "predict.hip", "greedy.hip", "synthetic.hip", "readbw.hip"]
# Measurement aids outside the kernel sources (whose digest ties the
# committed traffic records to the code they were taken on).
MEASURE = os.path.join(PKG, "measure")
MEASURE_SOURCES = ["lds_probe.hip"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libspecverify.so)")


def command(out: str = LIB, extra=()) -> list[str]:
    srcs = [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    srcs += [os.path.join(MEASURE, s) for s in MEASURE_SOURCES if os.path.exists(os.path.join(MEASURE, s))]
    return [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            "-I", INCLUDE, "-I", CSRC, *extra, "-o", out, *srcs]


def build(verbose: bool = False, out: str = LIB, defines: dict | None = None) -> str:
    """Compile the library; returns its path.  Always recompiles.  ``defines``
    sets tuning macros (SV_CHUNK, SV_STREAM_UNROLL, SV_TILES_PER_ITEM, ...)."""
    tmp = out + ".tmp"
    cmd = command(tmp, [f"-D{k}={v}" for k, v in (defines or {}).items()])
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    return out


def build_timeline(verbose: bool = False) -> str:
    """Compile the timeline measurement build (TIMELINE_LIB)."""
    return build(verbose, TIMELINE_LIB, {"SV_TIMELINE": 1})


def build_checks(verbose: bool = False) -> str:
    """Compile the checks build (CHECKS_LIB)."""
    return build(verbose, CHECKS_LIB, {"SV_CHECKS": 1})


if __name__ == "__main__":
    if "--timeline" in sys.argv:
        print(build_timeline(verbose="-v" in sys.argv))
    elif "--checks" in sys.argv:
        print(build_checks(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
