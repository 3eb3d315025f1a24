"""The C-ABI argument checks under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only, no GPU): fa_api.cpp built with g++ and both sanitizers
against stand-in launchers (tests/asan/stubs.cpp), driven through every entry
point's error paths and one passing call each (tests/asan/abi_driver.cpp)."""

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_31_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "asan")


def test_abi_checks_clean_under_sanitizers():
    gxx = shutil.which("g++")
    rocm_inc = "/opt/rocm/include"
    if not gxx or not os.path.isdir(rocm_inc):
        pytest.skip("g++ or the ROCm headers are missing")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "abi_driver")
        cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I", rocm_inc, "-I",
               os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "fa_api.cpp"),
               os.path.join(HERE, "stubs.cpp"), os.path.join(HERE, "abi_driver.cpp"), "-o", exe]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-4000:]
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
        run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        out = run.stdout + run.stderr
        assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
        assert run.returncode == 0 and "ok: 0 failures" in out, out[-4000:]
