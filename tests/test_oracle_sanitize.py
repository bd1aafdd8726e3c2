"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer:
tests/oracle_sanitize_driver.c calls every entry point of
oracle/fp8_oracle.c on small ragged inputs (NaN, Inf, zeros, subnormals,
values far past the formats' range, KV slots outside the cache) with
buffers of exactly the size each call may touch; the build stops at the
first report.  Host code only, built with gcc."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-O1", "-g", "-std=gnu11", "-fopenmp", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "fp8_oracle.c"), os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
           "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "ok" in r.stdout, (r.returncode, r.stderr[-4000:])
