"""Host-side checks of bench.py (no GPU): the operation count it divides by
time, its one-GPU contract, and its counter-summary guard."""
import json
import os
import subprocess
import sys

import bench
from tests.conftest import ROOT


def test_operation_count_matches_the_study_table():
    """GFLOPS x time in the study's benchmark table equals 2*M*N*K for every
    row, within the rounding of the printed times."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "study_benchmark_table.json")))
    ops = bench.flops(g["M"], g["N"], g["K"])
    dt = g["time_rounding_ms"]
    for row in g["rows"]:
        lo = ops / ((row["avg_ms"] + dt) * 1e-3) / 1e9
        hi = ops / ((row["avg_ms"] - dt) * 1e-3) / 1e9
        assert lo <= row["gflops"] <= hi, row
    # and a factor-of-two mistake (counting MACs) would not fit
    assert not (ops / 2 / (2.296e-3) / 1e9 > 7000)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_is_read_only_for_the_current_kernel_sources(tmp_path, monkeypatch):
    real = bench.kernel_source_hash()
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: real)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    f = prof / "traffic_int8_4096.txt"
    f.write_text("kernel_source_sha256_16: 0000000000000000\nhbm_bytes_per_launch_S2_direct: 123\n")
    assert bench.read_traffic("int8_4096", 2, "direct") is None
    f.write_text("kernel_source_sha256_16: %s\nhbm_bytes_per_launch_S2_direct: 123\n" % real)
    assert bench.read_traffic("int8_4096", 2, "direct") == 123.0
    assert bench.read_traffic("int8_4096", 3, "direct") is None


def test_kernel_hash_covers_the_kernel_sources():
    h1 = bench.kernel_source_hash()
    assert len(h1) == 16 and h1 == bench.kernel_source_hash()


def test_measured_ceiling_is_read_from_the_probe_output():
    """The committed ceiling_probe output gives one attainable rate per dtype
    and one for HBM, each below its datasheet peak."""
    for dt in ("i8", "f16", "bf16", "f32"):
        c = bench.measured_ceiling(dt, "mfma")
        assert c is not None and 0 < c <= bench.PEAK[dt], (dt, c)
    h = bench.measured_ceiling("bf16", "hbm")
    assert h is not None and 0 < h <= bench.HBM_PEAK_GBS


def test_kernel_hash_ignores_comments(tmp_path, monkeypatch):
    """Only a change of code, not of comments or spacing, changes the hash."""
    import shutil
    src = os.path.join(ROOT, "software_pipelined_tiled_02_amd", "csrc")
    root = tmp_path / "r"
    shutil.copytree(src, root / "software_pipelined_tiled_02_amd" / "csrc")
    monkeypatch.setattr(bench, "ROOT", str(root))
    h0 = bench.kernel_source_hash()
    f = root / "software_pipelined_tiled_02_amd" / "csrc" / "tile_layout.h"
    text = f.read_text()
    f.write_text("// a new comment\n/* and a block\n comment */\n" + text.replace("\n", "\n\n", 3))
    assert bench.kernel_source_hash() == h0
    f.write_text(text.replace("constexpr int kChunk = 16;", "constexpr int kChunk = 32;"))
    assert bench.kernel_source_hash() != h0
