"""Randomised checks of the library's host-side code (planners, prompt lookup,
greedy acceptance, the step planner over many plan / commit / release rounds):
tests/host_fuzz.cpp is compiled with g++ against include/ and linked to
libpgqa.so, and must report every part ok.  No GPU."""
import os
import shutil
import subprocess

import pytest

import paged_gqa_decode_head_amd as pg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_fuzz(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not available")
    exe = str(tmp_path / "host_fuzz")
    libdir = os.path.dirname(pg.LIB_PATH)
    cmd = [gxx, "-std=c++17", "-O2", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "host_fuzz.cpp"), "-L", libdir, "-lpgqa", f"-Wl,-rpath,{libdir}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe, "3000", "60"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    lines = r.stdout.splitlines()
    assert any(l.startswith("planners ok:") for l in lines), r.stdout
    assert any(l.startswith("step planner ok:") for l in lines), r.stdout
