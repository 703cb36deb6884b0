"""The ABI validation tests, re-run against a host-only build of the validation layer
(fa_api.cpp) compiled with AddressSanitizer and UndefinedBehaviorSanitizer.

The build links fa_api.cpp with stand-ins for the kernel launchers that abort when
reached (tests/sanitize/launch_stubs.cpp); no device code is involved.  The ABI tests run
in a child Python with the ASan runtime preloaded and FA_LIBRARY pointing at that build:
any out-of-bounds access, use of uninitialised memory the sanitizers track, undefined
behaviour or an argument block that reaches a launcher ends the child with an error.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "io_aware_tiled_10_amd", "csrc")
OUT_DIR = os.path.join(ROOT, "_build", "sanitize")
LIB = os.path.join(OUT_DIR, "libfa_host_asan.so")
ROCM = "/opt/rocm"


def build_sanitized_library() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    cmd = ["g++", "-std=c++17", "-shared", "-fPIC", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", f"{ROCM}/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "fa_api.cpp"), os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
           f"-L{ROCM}/lib", f"-Wl,-rpath,{ROCM}/lib", "-lamdhip64", "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return LIB


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(f"{ROCM}/include/hip/hip_runtime.h"),
                    reason="needs g++ and the ROCm headers")
def test_abi_validation_is_clean_under_asan_and_ubsan():
    lib = build_sanitized_library()
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    assert os.path.isabs(asan) and os.path.exists(asan), "libasan not found"
    env = dict(os.environ, LD_PRELOAD=asan, FA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "failed" not in r.stdout, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
