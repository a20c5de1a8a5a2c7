"""Host-side checks of bench.py's output contract (no GPU needed)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = r.stdout.strip().splitlines()[-1]
    assert "one GPU only" in json.loads(line)["error"]


def test_published_peaks():
    # MI355X dense peaks: bf16 2.5 PFLOP/s, fp8 5.0 PFLOP/s, HBM 8 TB/s
    assert bench.PEAK_BF16_TFLOPS == 2500.0
    assert bench.PEAK_FP8_TFLOPS == 5000.0
    assert bench.PEAK_HBM_GBS == 8000.0
    # the 8-bit-key tier: half the useful flops at each peak -> harmonic blend
    blend = 1.0 / (0.5 / bench.PEAK_FP8_TFLOPS + 0.5 / bench.PEAK_BF16_TFLOPS)
    assert bench.PEAK_FP8_TIER_TFLOPS == pytest.approx(blend, rel=1e-3)


def test_recorded_traffic_follows_the_kernel_hash(tmp_path, monkeypatch):
    h = bench.attn_kernel_hash()
    assert len(h) == 64
    good = tmp_path / "c.md"
    good.write_text(f"    kernel_sha256: {h}\n    traffic_bytes_per_launch: 123456\n")
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(good))
    assert bench.recorded_traffic("wan13_4step")[0] == 123456
    assert bench.recorded_traffic("wan13_5step")[0] is None
    stale = tmp_path / "s.md"
    stale.write_text("    kernel_sha256: " + "0" * 64 + "\n    traffic_bytes_per_launch: 123456\n")
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(stale))
    value, why = bench.recorded_traffic("wan13_4step")
    assert value is None and "changed" in why
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(tmp_path / "missing.md"))
    assert bench.recorded_traffic("wan13_4step")[0] is None
