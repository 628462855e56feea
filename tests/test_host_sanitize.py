"""The C ABI front end (q4_api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer.

gcc builds q4_api.cpp with tests/c/host_sanitize.cpp, whose stubs stand in for the
kernel launchers and the HIP runtime: no GPU and no device code are involved. The
program checks every entry point's argument validation, that a failing launch comes
back as Q4_ERR_HIP with the runtime's message (the stub launcher injects the failure),
that overflowing shapes are rejected, and the act-order permutation; any sanitizer
finding aborts it.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_api_host_checks_under_asan_ubsan(tmp_path):
    exe = tmp_path / "host_sanitize"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "w4a16_decode_amd", "csrc", "q4_api.cpp"),
           os.path.join(ROOT, "tests", "c", "host_sanitize.cpp"), "-o", str(exe)]
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, p.stdout + p.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks ok" in r.stdout
