"""The library's CPU code (T2 packer and unpacker, host checks of a step
description) built with AddressSanitizer and UndefinedBehaviorSanitizer and
run on edge cases: exactly sized buffers, the last weight out of range,
invalid codes, aliased and partly overlapping buffers, plan fingerprints.
g++ only, no GPU code (the sanitizers apply to host code)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "packed_weight_gemv_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_code_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "host_sanitize"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I" + CSRC,
           os.path.join(ROOT, "tests", "native", "host_sanitize.cpp"),
           os.path.join(CSRC, "pack.cpp"), os.path.join(CSRC, "blob.cpp"), os.path.join(CSRC, "errors.cpp"),
           os.path.join(CSRC, "validate.cpp"),
           "-o", str(exe), "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "host checks ok" in r.stdout, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
