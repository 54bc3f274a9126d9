"""The host C ABI layer (csrc/api.cpp) built with AddressSanitizer and
UndefinedBehaviorSanitizer by g++, against a host stand-in for the HIP runtime
and recording launch stubs (tests/hoststub, tests/host_abi_driver.cpp): every
entry point with valid and invalid arguments, sizes at the int32 limit, and
the debug index checks of cu_seqlens and block tables.  Any sanitizer report
aborts the run; a wrong status is a mismatch."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_abi_under_asan_ubsan(tmp_path):
    exe = tmp_path / "host_abi"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-Wall", "-Werror",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "tests", "hoststub"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "host_abi_driver.cpp"),
           os.path.join(ROOT, "attention_attn_fwd_10_amd", "csrc", "api.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env)
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-2000:]
    assert r.stdout.strip().endswith("mismatches 0")
