"""Sanitizer builds of the host code, run on the CPU (no GPU needed).

  - The oracle (plain C), built with the address and undefined-behaviour sanitizers and
    driven through every entry point on small seeded inputs, valid and invalid
    (tests/sanitize/oracle_driver.c).
  - The verify library's host side: spec_verify.hip built with both sanitizers on the
    host pass only (each -fsanitize= placed after -Xarch_host, so the gfx950 code is built
    as usual), linked into a driver that calls every entry point with arguments the host
    must reject before any launch (tests/sanitize/abi_driver.cpp).

Each build goes to a temporary directory; a report from either sanitizer fails the test.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc is not available")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
          "-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
          "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
          os.path.join(ROOT, "oracle", "spec_oracle.c"), os.path.join(HERE, "oracle_driver.c"),
          "-lm", "-o", exe])
    r = _run([exe], env=dict(ENV, OMP_NUM_THREADS="2"))
    assert "all calls checked" in r.stdout


def test_host_abi_under_address_and_undefined_sanitizers(tmp_path):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc is not available")
    exe = str(tmp_path / "abi_driver")
    src = os.path.join(ROOT, "lossless_rejection_sampling_verify_amd", "csrc", "spec_verify.hip")
    _run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "include"), src, os.path.join(HERE, "abi_driver.cpp"),
          "-o", exe], timeout=900)
    # the HIP runtime's own allocations outlive main: leak reports are for our code only,
    # and it allocates nothing, so leak checking is off here
    r = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1"))
    assert "all argument checks passed" in r.stdout
