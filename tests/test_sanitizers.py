"""The CPU oracle and the library's host code built with AddressSanitizer
and UndefinedBehaviorSanitizer (host code only; no device code is
instrumented) and run on the CPU: see tests/host/sanitize_*.  Any report of
either sanitizer fails the test."""
import os
import shutil
import subprocess

import pytest

from tests.conftest import ROOT

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    out = p.stdout + p.stderr
    assert p.returncode == 0 and "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    return out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "san_oracle")
    subprocess.run(["gcc", "-std=c99", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", os.path.join(ROOT, "tests", "host", "sanitize_oracle.c"),
                    os.path.join(ROOT, "oracle", "oracle_gemm.c"), "-o", exe, "-lm"], check=True)
    assert "OK" in _run(exe)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_host_abi_under_sanitizers(tmp_path):
    exe = str(tmp_path / "san_abi")
    csrc = os.path.join(ROOT, "software_pipelined_tiled_02_amd", "csrc")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I" + os.path.join(ROOT, "include"), "-I" + csrc,
                    os.path.join(csrc, "abi.hip"), os.path.join(ROOT, "tests", "host", "sanitize_abi.cpp"),
                    "-o", exe], check=True)
    assert "OK" in _run(exe)
