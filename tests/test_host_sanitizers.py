"""The host code of libtq (tq_host.cpp: codebooks, tq_prepare, argument checks,
workspace plans, dispatch) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, with the kernel launchers replaced by host stubs
(tests/sanitize/launch_stubs.cpp), and driven through every C entry point by
tests/sanitize/host_driver.cpp.  No GPU code is built or run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_host_code_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("g++ or the HIP headers are missing")
    exe = str(tmp_path / "host_driver")
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include",
           f"-I{ROOT}/kv_cache_online_amd/csrc",
           os.path.join(ROOT, "kv_cache_online_amd", "csrc", "tq_host.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert "host paths ok" in r.stdout
