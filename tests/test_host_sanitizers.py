"""The C-ABI layer built for the host alone (launchers replaced by stand-ins) under AddressSanitizer and
UBSan, driven through every host-side check by tests/host_check/abi_driver.cpp.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_self_attention_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_check")


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "abi_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "mask_sizes.cpp"),
           os.path.join(HERE, "launch_stubs.cpp"), os.path.join(HERE, "abi_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "host ABI checks passed" in r.stdout
