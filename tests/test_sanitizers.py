"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the host code.

Two check programs under ``tests/sanitize/`` are compiled with
``-fsanitize=address,undefined -fno-sanitize-recover=all`` and run:

* ``oracle_check.c`` links ``oracle/mla_oracle.c`` and calls every oracle
  function on small ragged inputs, including the padding, repeat, empty-row
  and out-of-range paths (leak checking on).
* ``api_check.cpp`` links ``sparse_mla_amd/csrc/mla_api.cpp`` -- the host
  argument checks, plans and workspace layouts of every C-ABI entry point --
  against stub launchers that record the kernel arguments instead of
  launching, and drives it with valid, invalid and extreme arguments.

Host code only: nothing here is built for or runs on a GPU.
"""
import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-O1"]


def _build_and_run(cmd, exe, expect):
    if shutil.which(cmd[0]) is None:
        pytest.skip(f"{cmd[0]} not available")
    b = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
    r = subprocess.run([str(exe)], cwd=ROOT, capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert expect in r.stdout
    assert "runtime error" not in r.stderr


def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_check"
    _build_and_run(["gcc", *SAN, "-fopenmp", "tests/sanitize/oracle_check.c", "oracle/mla_oracle.c",
                    "-lm", "-o", str(exe)], exe, "oracle sanitizer check: ok")


def test_api_host_checks_under_sanitizers(tmp_path):
    exe = tmp_path / "api_check"
    _build_and_run(["g++", "-std=c++17", *SAN, "-Iinclude", "-Isparse_mla_amd/csrc",
                    "tests/sanitize/api_check.cpp", "sparse_mla_amd/csrc/mla_api.cpp", "-o", str(exe)],
                   exe, "api sanitizer check: ok")
