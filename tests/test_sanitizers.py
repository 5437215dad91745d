"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the CPU code (CPU only).

Two separate programs, so the oracle and the library's host code are never
linked together: the oracle with its driver, and the host part of the C ABI
(host.cpp) with its own. Any sanitizer report aborts the program
(-fno-sanitize-recover), which fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1",
       "-ffp-contract=off"]


def _run(cmd, exe, tmp_path):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    # verify_asan_link_order=0: the environment may preload a library ahead of
    # the ASan runtime; that does not affect what ASan checks in this program.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, cwd=tmp_path, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    cmd = ["gcc", "-std=c11", *SAN, "-fopenmp", os.path.join(ROOT, "oracle", "bitlinear_oracle.c"),
           os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-o", exe, "-lm"]
    _run(cmd, exe, tmp_path)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_abi_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_san")
    cmd = ["g++", "-std=c++17", *SAN, os.path.join(ROOT, "bitlinear_amd", "csrc", "host.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp"), "-o", exe]
    _run(cmd, exe, tmp_path)
