"""Host-side logic of bench.py (no GPU): the counter-summary parser that
fills roofline.traffic, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_traffic_parser(tmp_path):
    f = tmp_path / "t.txt"
    f.write_text("# comment: with a colon\ngemm_bf16_hip_sha256_16: abc123\n"
                 "hbm_bytes_per_launch: 12345\n")
    assert bench.measured_traffic(str(f), "abc123") == 12345.0
    assert bench.measured_traffic(str(f), "other") is None      # stale: kernel changed
    assert bench.measured_traffic(str(tmp_path / "missing.txt"), "abc123") is None
    f.write_text("gemm_bf16_hip_sha256_16: abc123\nhbm_bytes_per_launch: 12345\n"
                 "shader_clock_ghz: 1.8\n")
    assert bench.measured_counters(str(f), "abc123")["shader_clock_ghz"] == 1.8
    assert bench.measured_counters(str(f), "other") is None


def test_committed_traffic_files_parse():
    # each committed summary names the kernel source it was taken on; the
    # current GEMM source is the one they were taken on
    for path in bench.TRAFFIC_FILES.values():
        kv = dict(l.split(":", 1) for l in open(path) if ":" in l and not l.startswith("#"))
        h = kv["gemm_bf16_hip_sha256_16"].strip()
        assert bench.measured_traffic(path, h) > 0
        assert h == bench.kernel_source_hash(), path
        assert float(kv["hbm_bytes_per_launch"]) > float(kv["algorithmic_bytes_per_launch"])
        c = bench.measured_counters(path, h)
        assert 1.0 < c["shader_clock_ghz"] <= 2.4 and 0.0 < c["mfma_busy"] <= 1.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "single" in r.stderr
