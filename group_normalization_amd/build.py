"""Build libskipnorm.so, the HIP library behind the C ABI, for gfx950.

Compiles every source under ``csrc/`` with hipcc (one process per source, in
parallel) and links them into ``group_normalization_amd/libskipnorm.so``.
Runs on a machine without a GPU: hipcc cross-compiles for gfx950.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libskipnorm.so")
# Measurement build: the same library with SN_PHASE_TRACE, whose single-launch
# SkipGroupNorm kernels record per-workgroup phase timestamps in a tail of
# the workspace (read by `bench.py --phases`).  Never loaded by the package.
TRACE_BUILD_DIR = os.path.join(PKG, "_build_phase_trace")
TRACE_LIB_PATH = os.path.join(PKG, "libskipnorm_phase_trace.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["skipnorm_api.cpp", "ssln.hip", "gated.hip", "sgn.hip", "sgn_nhwc.hip", "copy.hip"]

# -ffp-contract=off: no implicit FMA, so the float32 arithmetic is exactly the
# operations written (explicit FMAs are spelled __builtin_fmaf).
# -packed-fp32-ops: no v_pk_*_f32 generation.
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def _compile(src: str, build_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the GPU-only feature flag and says so;
    # that line is expected, anything else is shown.
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build(jobs: int | None = None, phase_trace: bool = False) -> str:
    """Compile and link the library (or, with phase_trace, the measurement
    build); returns its path."""
    build_dir, lib_path = (TRACE_BUILD_DIR, TRACE_LIB_PATH) if phase_trace else (BUILD_DIR, LIB_PATH)
    extra = ["-DSN_PHASE_TRACE"] if phase_trace else []
    os.makedirs(build_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), SOURCES))
    tmp = lib_path + ".tmp"
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                   check=True)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(phase_trace="--phase-trace" in sys.argv[1:]))
