"""The C ABI from plain C: include/ecco.h compiles as C99 with warnings as
errors, a C program links against the built library, and its host-side calls
(tables, tensor scale, argument checks of the device calls) behave as the
header declares.  Host only; skipped when the library is not built."""

import os
import shutil
import subprocess

import pytest

import entropy_coded_group_amd as ecco

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.skipif(not os.path.exists(ecco.library_path), reason="libecco.so is not built")
def test_c_program_links_and_calls_the_host_side(tmp_path):
    exe = str(tmp_path / "abi_host")
    libdir = os.path.dirname(ecco.library_path)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_host.c"), "-o", exe, libdir + "/libecco.so",
           "-Wl,-rpath," + libdir, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
