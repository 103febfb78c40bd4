"""Host-side logic of bench.py, on the CPU: the one-GPU refusal, the rule that
a committed traffic summary counts only when it was taken on the current kernel
source, and the vendor-GEMM comparison reporting its own failure."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.fixture()
def fake_root(tmp_path, monkeypatch):
    csrc = tmp_path / "post_w8a8_quantized_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("kernel source v1\n")
    (csrc / "zq_device.h").write_text("helpers\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def write_summary(root, src_hash, total):
    (root / "profiles" / "traffic_k_wl.txt").write_text(
        "# HBM traffic per launch of k\n"
        f"source_hash = {src_hash}\n"
        "launches = 10\n"
        f"hbm_bytes_per_launch = {total}\n")


def test_traffic_read_only_for_the_current_source(fake_root):
    h = bench.kernel_source_hash(["k.hip", "zq_device.h"])
    assert h == bench.kernel_source_hash(["k.hip", "zq_device.h"])
    write_summary(fake_root, h, 123456)
    assert bench.read_traffic("k", "wl", h) == 123456.0
    # the kernel changes after the counters were taken: the figure no longer counts
    (fake_root / "post_w8a8_quantized_amd" / "csrc" / "k.hip").write_text("kernel source v2\n")
    h2 = bench.kernel_source_hash(["k.hip", "zq_device.h"])
    assert h2 != h
    assert bench.read_traffic("k", "wl", h2) is None
    # a shared header counts as part of the source
    write_summary(fake_root, h2, 7)
    (fake_root / "post_w8a8_quantized_amd" / "csrc" / "zq_device.h").write_text("helpers v2\n")
    assert bench.read_traffic("k", "wl", bench.kernel_source_hash(["k.hip", "zq_device.h"])) is None


def test_missing_or_malformed_summary(fake_root):
    assert bench.read_traffic("k", "other", "abc") is None
    (fake_root / "profiles" / "traffic_k_wl.txt").write_text("source_hash = abc\n")
    assert bench.read_traffic("k", "wl", "abc") is None


def test_min_traffic_leaves_out_the_codes_round_trip():
    class Decode:
        M, K = 16, 28672
    # the decode layer's bytes: X fp16, codes and scales out and back in, the
    # packed weights with their group scales, Y fp16 (no bias)
    X, codes, W, sw, Y = 16 * 28672 * 2, 16 * 28672 + 4 * 16, 8192 * 28672, 4 * 64, 16 * 8192 * 2
    layer = X + 2 * codes + W + sw + Y
    got = bench.min_traffic(Decode, {"unit": "GB/s", "bytes_layer": layer, "ms_step": 0.04})
    assert got["min_traffic_bytes"] == X + W + sw + Y
    assert abs(got["min_traffic_GBps"] - (X + W + sw + Y) / 40e-6 / 1e9) < 0.1
    assert bench.min_traffic(Decode, {"unit": "TOPS", "bytes_layer": layer, "ms_step": 0.04}) == {}


def test_library_reference_failure_is_reported_not_raised(monkeypatch):
    """The vendor-GEMM comparison is context only: if torch cannot run it, the
    benchmark line carries the reason instead of failing."""
    class Cuda:
        synced = 0

        @classmethod
        def synchronize(cls):
            cls.synced += 1

    class Torch:
        cuda = Cuda

    def boom(*a, **k):
        raise RuntimeError("_int_mm is not supported for this shape")

    monkeypatch.setattr(bench, "library_leg", boom)
    out = bench.guarded_library_leg(Torch, None, {}, None, None)
    assert out == {"error": "RuntimeError: _int_mm is not supported for this shape"}
    assert Cuda.synced == 1

    monkeypatch.setattr(bench, "library_leg", lambda *a: {"library_int32_us": 1.0})
    assert bench.guarded_library_leg(Torch, None, {}, None, None) == {"library_int32_us": 1.0}
