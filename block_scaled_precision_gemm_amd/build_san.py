"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the
library, for the CPU ABI tests.

    python -m block_scaled_precision_gemm_amd.build_san

The host sources (argument validation, planning, dispatch, timing) are
compiled with g++ and both sanitizers; the device objects are the ones the
regular build left in _build/ (no device code is ever sanitized).  The
result is _build/libbsmm_san.so, loaded in place of libbsmm.so when
BSMM_LIB_PATH names it, in a Python started with the ASan runtime
preloaded (see ``sanitizer_env``).
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

from .build import CSRC, HOST_SOURCES, INCLUDE, OBJDIR

SAN_LIB = os.path.join(OBJDIR, "libbsmm_san.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer"]


def device_objects():
    """The regular build's device objects (kernels, packing, quantisers,
    probe, scratch); empty if it has not run."""
    objs = sorted(glob.glob(os.path.join(OBJDIR, "bsmm_kernels_*.o")))
    for name in ("bsmm_pack.o", "bsmm_quant.o", "bsmm_probe.o", "bsmm_scratch.o"):
        objs.append(os.path.join(OBJDIR, name))
    return [o for o in objs if os.path.exists(o)]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"sanitizer build failed: {cmd[-1]}")


def build_sanitized() -> str:
    dev = device_objects()
    if len(dev) < 5:
        raise RuntimeError("the regular build has not run: no device objects in " + OBJDIR)
    host = []
    for s in HOST_SOURCES:
        o = os.path.join(OBJDIR, s + ".san.o")
        _run(["g++", "-O1", "-g", "-std=c++17", "-fPIC", *SAN_FLAGS, "-I" + INCLUDE,
              "-I" + CSRC, "-I" + os.path.join(ROCM, "include"), "-D__HIP_PLATFORM_AMD__",
              "-Wall", "-Wno-unused-function", "-c", os.path.join(CSRC, s), "-o", o])
        host.append(o)
    tmp = SAN_LIB + ".tmp"
    _run(["g++", "-shared", *SAN_FLAGS, *host, *dev, "-L" + os.path.join(ROCM, "lib"),
          "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", tmp])
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def sanitizer_env(base=None):
    """Environment for a Python process that loads the sanitized library:
    the ASan runtime preloaded (Python itself is not instrumented), leak
    checking off (the interpreter keeps its allocations at exit), any
    report fatal."""
    env = dict(os.environ if base is None else base)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["BSMM_LIB_PATH"] = SAN_LIB
    return env


if __name__ == "__main__":
    print("built", build_sanitized())
