"""The library's host C++ (entropy_coded_group_amd/csrc/ecco_tables.cpp and
ecco_train.cpp) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer and driven by tests/c/host_sanitize.cpp (training,
table round trips, degenerate samples).  Host only; no device code is built."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "entropy_coded_group_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-pthread", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "c", "host_sanitize.cpp"), os.path.join(CSRC, "ecco_train.cpp"),
           os.path.join(CSRC, "ecco_tables.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
