"""The C-ABI tests again, against the library built with AddressSanitizer
and UndefinedBehaviorSanitizer on its host code (argument validation, plan
selection, the dispatch table, the override and timing state).  The
sanitized build reuses the regular build's device objects; the tests run in
a child Python with the ASan runtime preloaded, and any sanitizer report
aborts it."""

import os
import subprocess
import sys

import pytest

from block_scaled_precision_gemm_amd import build_san

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHECK_LOADED = r"""
import ctypes, sys
import block_scaled_precision_gemm_amd as bsmm
bsmm.load()
maps = open("/proc/self/maps").read()
assert "libbsmm_san.so" in maps and "libbsmm.so" not in maps.replace("libbsmm_san.so", ""), \
    "the sanitized library is not the one loaded"
ctypes.CDLL(None).__asan_init          # the ASan runtime is in the process
print("sanitized library loaded:", bsmm.lib_path)
"""


@pytest.fixture(scope="module")
def san_env():
    if len(build_san.device_objects()) < 5:
        pytest.skip("the regular build has not run (no device objects)")
    build_san.build_sanitized()
    env = build_san.sanitizer_env()
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    return env


def _run(env, args):
    r = subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_sanitized_library_is_the_one_loaded(san_env):
    assert "sanitized library loaded" in _run(san_env, ["-c", CHECK_LOADED])


def test_abi_suite_under_asan_and_ubsan(san_env):
    out = _run(san_env, ["-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                         os.path.join("tests", "test_abi.py")])
    assert " passed" in out and " failed" not in out, out[-2000:]
