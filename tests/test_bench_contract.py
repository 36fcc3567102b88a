"""CPU checks of bench.py's reporting contract: the one-GPU refusal, the
roofline fields, and the rule that a committed traffic figure is reported only
for the kernel sources it was measured on."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_roofline_fields():
    m = bench.roofline_mfma(1000.0, traffic=123)
    assert m == {"bound": "mfma", "achieved": 1000.0, "peak": 2500.0, "unit": "TFLOP/s",
                 "frac": 0.4, "traffic": 123}
    h = bench.roofline_hbm(6000.0)
    assert h["bound"] == "hbm" and h["unit"] == "GB/s" and h["peak"] == 8000.0
    assert h["frac"] == 0.75 and h["traffic"] is None


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    csrc = tmp_path / "tiled_attention_09_amd" / "csrc"
    csrc.mkdir(parents=True)
    f = csrc / "k.hip"
    f.write_text("int a = 1;  // one\n\nint b = 2;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h1 = bench.kernel_source_hash(("k.hip",))
    f.write_text("// a new comment\nint a = 1;\nint b = 2;   \n")
    assert bench.kernel_source_hash(("k.hip",)) == h1
    f.write_text("int a = 1;\nint b = 3;\n")
    assert bench.kernel_source_hash(("k.hip",)) != h1


def test_traffic_reported_only_for_the_measured_kernel(tmp_path, monkeypatch):
    csrc = tmp_path / "tiled_attention_09_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("int a = 1;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    names = ("k.hip",)
    summary = tmp_path / "traffic.json"
    summary.write_text(json.dumps({"workload": "w", "bytes_per_launch": 42,
                                   "kernel_source_sha256": bench.kernel_source_hash(names)}))
    assert bench.measured_traffic("w", str(summary), names) == 42
    assert bench.measured_traffic("other", str(summary), names) is None
    (csrc / "k.hip").write_text("int a = 2;\n")
    assert bench.measured_traffic("w", str(summary), names) is None
    assert bench.measured_traffic("w", str(tmp_path / "missing.json"), names) is None


@pytest.mark.parametrize("key,want", [("fwd", 7), ("bwd", None)])
def test_traffic_of_one_path_in_a_multi_path_summary(tmp_path, monkeypatch, key, want):
    csrc = tmp_path / "tiled_attention_09_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("int a = 1;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    names = ("k.hip",)
    summary = tmp_path / "paths.json"
    summary.write_text(json.dumps({"workload": "w", "paths": {
        "fwd": {"bytes_per_launch": 7, "kernel_source_sha256": bench.kernel_source_hash(names)}}}))
    assert bench.measured_traffic("w", str(summary), names, key=key) == want
