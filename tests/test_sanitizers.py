"""Host AddressSanitizer / UndefinedBehaviorSanitizer runs (CPU only).

Builds the oracle (oracle/attn_oracle.c) and the library's host code
(split_kv_paged_amd/csrc/attn_api.cpp: planners, validation, the paged-input
checker) with gcc/g++ -fsanitize=address,undefined and no recovery, each with
a driver under tests/sanitize/, and runs them.  A sanitizer report or a
failed driver check ends the driver with a non-zero status.  No GPU code is
built: the HIP runtime is linked for its symbols only, and the launch
functions are stubs that abort if reached.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _run(exe, detect_leaks):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=%d:abort_on_error=0" % detect_leaks,
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, "status %d\n%s\n%s" % (r.returncode, r.stdout, r.stderr[-4000:])
    assert "ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.check_call(["gcc", "-std=c99", "-D_DEFAULT_SOURCE", "-Wall", "-pthread"] + SAN +
                          [os.path.join(ROOT, "oracle", "attn_oracle.c"),
                           os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                           "-o", exe, "-lm"])
    _run(exe, detect_leaks=1)


@pytest.mark.skipif(shutil.which("g++") is None or
                    not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")),
                    reason="g++ or HIP headers not found")
def test_host_api_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "api_driver")
    # leak checking off: the HIP runtime's own start-up allocations are not ours
    subprocess.check_call(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__",
                           "-I" + os.path.join(ROCM, "include"),
                           "-I" + os.path.join(ROOT, "include"),
                           "-I" + os.path.join(ROOT, "split_kv_paged_amd", "csrc")] + SAN +
                          [os.path.join(ROOT, "split_kv_paged_amd", "csrc", "attn_api.cpp"),
                           os.path.join(ROOT, "tests", "sanitize", "api_driver.cpp"),
                           "-o", exe, "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
                           "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    _run(exe, detect_leaks=0)
