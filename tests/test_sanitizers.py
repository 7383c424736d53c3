"""Host code under the address and undefined-behaviour sanitizers (CPU only).

- The C oracle, compiled with gcc -fsanitize=address,undefined together with
  tests/sanitize/oracle_driver.c, which cuts every row to its exact valid
  length in its own heap block (a read past the prefix is a reported heap
  overflow) and checks each result against a brute-force rank count.
- The C ABI host code (topk_api.hip built with host-only sanitizers, linked
  with the normal kernel object) driven by tests/sanitize/api_driver.cpp
  through every entry point's host-checkable argument errors; with no GPU, a
  valid configuration stops at the device query.
A sanitizer report fails the run (-fno-sanitize-recover=all).
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(exe: str) -> subprocess.CompletedProcess:
    env = dict(os.environ)
    # the HIP runtime keeps allocations for the life of the process
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    return subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.check_call(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "oracle_topk.c"),
                           os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm", "-o", exe])
    r = _run(exe)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle sanitizer checks passed" in r.stdout


def test_c_abi_host_code_under_asan_ubsan():
    from sparse_attention_indexer_amd import build
    if not os.path.exists(build.CLANGXX):
        pytest.skip("ROCm clang++ not found")
    exe = build.build_api_sanitizer_driver()
    r = _run(exe)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "api sanitizer checks passed" in r.stdout
