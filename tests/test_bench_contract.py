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


def test_rollout_driver_fill_masks_match_the_oracle():
    """The bench's rollout driver occupies slots as the tick composition says."""
    import oracle
    for S in (2, 4, 5):
        for t in range(3 * S):
            assert bench.active_slots(t, S) == oracle.active_mask_for_tick(t, S), (S, t)


def test_power_window_medians_and_fallbacks(monkeypatch):
    """Power and clock summary from a stand-in metrics library: medians over
    the samples, per XCD, invalid clock entries dropped; a missing library or
    an empty table gives an error note instead of failing the bench."""
    import types

    readings = iter([(1390, [1700, 1800, 65535]), (1380, [1720, 1760, 65535]),
                     (1400, [1710, 1790, 65535])] + [(1395, [1705, 1795, 65535])] * 100)
    fake = types.SimpleNamespace(
        amdsmi_init=lambda: None,
        amdsmi_get_processor_handles=lambda: ["gpu0"],
        amdsmi_get_gpu_metrics_info=lambda h: dict(zip(("current_socket_power", "current_gfxclks"),
                                                       next(readings))),
        amdsmi_shut_down=lambda: None)
    monkeypatch.setitem(sys.modules, "amdsmi", fake)
    import time
    ticks = []

    def step():
        ticks.append(1)
        time.sleep(0.001)
    r = bench.power_window(step, seconds=0.8, sync=lambda: None)
    assert r["samples"] >= 2 and r["ticks"] == len(ticks) > 0
    assert len(r["gfx_clk_mhz_per_xcd"]) == 2           # the 65535 placeholder dropped
    assert 1380 <= r["socket_power_w"] <= 1400
    assert 1700 <= r["gfx_clk_mhz_per_xcd"][0] <= 1720 and 1760 <= r["gfx_clk_mhz_per_xcd"][1] <= 1800
    assert r["gfx_clk_mhz_mean"] == pytest.approx(sum(r["gfx_clk_mhz_per_xcd"]) / 2, abs=0.1)

    def broken_init():
        raise RuntimeError("driver not loaded")
    monkeypatch.setitem(sys.modules, "amdsmi", types.SimpleNamespace(amdsmi_init=broken_init))
    assert "error" in bench.power_window(lambda: None, seconds=0.1, sync=lambda: None)

    empty = types.SimpleNamespace(
        amdsmi_init=lambda: None, amdsmi_get_processor_handles=lambda: ["gpu0"],
        amdsmi_get_gpu_metrics_info=lambda h: {"current_socket_power": "N/A"},
        amdsmi_shut_down=lambda: None)
    monkeypatch.setitem(sys.modules, "amdsmi", empty)
    assert "error" in bench.power_window(lambda: None, seconds=0.6, sync=lambda: None)
