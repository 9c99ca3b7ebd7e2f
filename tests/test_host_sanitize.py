"""The host-side packer (moe_token_int8_amd/csrc/w4a8_host.cpp) built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven through every entry point, format and error path by
tests/host_sanitize_driver.cpp.  Host code only (the packer has no device code); runs on the CPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_packer_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-pthread", "-I" + os.path.join(ROOT, "moe_token_int8_amd", "csrc"),
           os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"),
           os.path.join(ROOT, "moe_token_int8_amd", "csrc", "w4a8_host.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failed checks" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
