"""CPU checks of the measurement helpers in bench.py: the useful-work formulas
against brute force and the workloads' stated figures, the traffic lookup,
and the one-GPU contract of the command line."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import swa_inputs as si  # noqa: E402


@pytest.mark.parametrize("T,W", [(1, 1), (5, 1), (5, 3), (8, 4), (16, 16), (16, 40), (37, 9)])
def test_band_pairs_is_the_count_of_visible_pairs(T, W):
    brute = sum(1 for i in range(T) for j in range(T) if j <= i and i - j < W)
    assert bench.band_pairs(T, W) == brute


def test_prefill_flops_of_the_headline_layer():
    w = si.WORKLOADS[bench.PREFILL]
    # 4 D flops per visible pair: 25,167,872 pairs per head at T 8192, W 4096
    assert bench.band_pairs(w.T, w.W) == 25_167_872
    assert bench.prefill_flops(w.B, w.H, w.T, w.D, w.W) == 412_350_414_848


def test_decode_bytes_of_the_decode_workload():
    w = si.WORKLOADS[bench.DECODE]
    # k and v of W slots for every (stream, head), plus q and out, in bf16
    assert bench.decode_bytes(w.S, w.H, w.D, w.W) == 2 * 256 * 32 * 4096 * 128 * 2 + 2 * 256 * 32 * 128 * 2


def test_traffic_lookup_requires_the_same_kernel_source(tmp_path, monkeypatch):
    p = tmp_path / "k_traffic.txt"
    p.write_text("# header\nkernel_source_sha: abc\nhbm_bytes_per_launch: 123456\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.read_traffic("k_traffic.txt", "abc") == 123456.0
    assert bench.read_traffic("k_traffic.txt", "abd") is None
    assert bench.read_traffic("missing.txt", "abc") is None


def test_source_sha_changes_with_the_source(tmp_path, monkeypatch):
    a = tmp_path / "a.hip"
    a.write_text("x")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    s1 = bench.source_sha(["a.hip"])
    a.write_text("y")
    assert bench.source_sha(["a.hip"]) != s1


def test_more_than_one_gpu_is_refused_before_touching_a_device():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
