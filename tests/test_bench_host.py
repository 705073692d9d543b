"""Host logic of bench.py (no GPU): the one-GPU contract, the weight-copy
rotation that keeps every timed launch reading HBM, and the measured-traffic
record that must go null when the kernel source changes."""

import argparse
import os
import subprocess
import sys

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_weight_bytes_formula():
    # codes + E4M3 block scales + the f32 global scale
    assert bench.weight_bytes(4096, 4096) == 4096 * 2048 + 4096 * 256 + 4
    assert bench.weight_bytes(51200, 5120) == 147_456_004


def test_rotation_covers_the_caches():
    args = argparse.Namespace(rotate_mb=576.0)
    for c in W.qwen3_32b_cases():
        n = bench.n_copies(args, c)
        assert n >= 2
        # 2 x (256 MB Infinity Cache + 32 MB L2)
        assert n * bench.weight_bytes(c.N, c.K) >= 576e6, c.name
        assert (n - 1) * bench.weight_bytes(c.N, c.K) < 576e6, c.name  # and no more copies than needed


def test_traffic_record_is_tied_to_the_kernel_source(monkeypatch):
    rec = dict(bench.GEMV_TRAFFIC)
    monkeypatch.setattr(bench, "GEMV_TRAFFIC", dict(rec, sha256="0" * 64))
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "GEMV_TRAFFIC", dict(rec, source="no/such/file.hip"))
    assert bench.measured_traffic() is None
