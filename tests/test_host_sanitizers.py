"""The library's host logic under AddressSanitizer and UndefinedBehaviorSanitizer.

``tests/host_check/host_api_check.cpp`` drives every host entry point (argument checks,
LPT and placements, mask helpers, and the cost / forward / backward descriptor and
workspace layouts over hundreds of random chunk tables) with the kernel launchers
replaced by checking stubs; it is compiled together with the library's host sources by
g++ with both sanitizers and must run clean.  No GPU is involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_cross_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_logic_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_api_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "layout.cpp"),
           os.path.join(ROOT, "tests", "host_check", "host_api_check.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, (run.stdout + run.stderr)[-6000:]
    assert "host check OK" in run.stdout
