"""Host check of the LDS tile layout shared by the kernels (no GPU): the XOR
swizzle is a per-row bijection and makes the MFMA fragment reads free of bank
conflicts under both LDS bank models; see tests/host/check_tile_layout.cpp."""
import os
import subprocess
import tempfile

from tests.conftest import ROOT


def test_tile_layout_host_check():
    src = os.path.join(ROOT, "tests", "host", "check_tile_layout.cpp")
    inc = os.path.join(ROOT, "software_pipelined_tiled_02_amd", "csrc")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "check")
        subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-I", inc, src, "-o", exe], check=True)
        r = subprocess.run([exe], capture_output=True, text=True)
        print(r.stdout)
        assert r.returncode == 0, r.stdout
        assert r.stdout.strip().endswith("OK")
