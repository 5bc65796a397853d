"""Build libbsmm.so in-tree with hipcc for gfx950.

    python -m block_scaled_precision_gemm_amd.build

Host sources (validation, dispatch) are plain C++; the kernels are HIP.  All
device code is compiled with packed-fp32 instructions disabled.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbsmm.so")
OBJDIR = os.path.join(PKG, "_build")
ARCH = "gfx950"

HOST_SOURCES = ["bsmm_api.cpp", "bsmm_tuned.cpp", "bsmm_variants.cpp", "bsmm_timing.cpp"]
HIP_SOURCE = "bsmm_kernels.hip"
# The kernel source is compiled once per (operation, output type) pair, in
# parallel; each object holds that pair's kernels for every configuration.
#   ops: 0 int8 rowwise, 1 fp8 blockwise, 2 fp8 mx, 3 fp8 scaled_mm, 4 fp8 mx32,
#        5 fp8 groupwise;
#   outputs: 0 i32, 1 f32, 2 bf16, 3 e4m3
KERNEL_UNITS = [(0, 0), (0, 1), (0, 2), (1, 1), (1, 2), (2, 1), (2, 2), (3, 1), (3, 2), (3, 3),
                (4, 1), (4, 2), (5, 1), (5, 2)]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC, "-Wall",
          "-Wno-unused-function"]
HIP_FLAGS = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-munsafe-fp-atomics"]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.exists(c) or c == "hipcc":
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"compile failed: {cmd[-1]}")
    return r


def build(verbose: bool = False) -> str:
    """Compile every source and link libbsmm.so; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    for s in HOST_SOURCES:
        o = os.path.join(OBJDIR, s + ".o")
        jobs.append([hipcc, *COMMON, "-c", os.path.join(CSRC, s), "-o", o])
    for op, out in KERNEL_UNITS:
        o = os.path.join(OBJDIR, f"bsmm_kernels_{op}_{out}.o")
        jobs.append([hipcc, *COMMON, *HIP_FLAGS, f"-DBSMM_TU_OP={op}",
                     f"-DBSMM_TU_OUT={out}", "-x", "hip", "-c",
                     os.path.join(CSRC, HIP_SOURCE), "-o", o])
    for src in ("bsmm_pack.hip", "bsmm_quant.hip", "bsmm_probe.hip", "bsmm_scratch.hip"):
        o = os.path.join(OBJDIR, src.replace(".hip", ".o"))
        jobs.append([hipcc, *COMMON, *HIP_FLAGS, "-x", "hip", "-c",
                     os.path.join(CSRC, src), "-o", o])
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(_run, jobs))
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
