"""Host-side logic of bench.py (no GPU): the clock sampler's window
statistics, the sampler's behaviour without a GPU driver, and the one-GPU
guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _sample(t, xcd=1500.0, cur=0xFFFF, avg=1490, power=1380, hot=80, e_uj=0.0, thr=0xFFFFFFFF):
    return (t, cur, xcd, avg, power, hot, e_uj, thr)


def test_refreshes_keep_the_samples_where_the_table_changed():
    s = [_sample(0.0, xcd=100.0), _sample(0.001, xcd=100.0), _sample(0.9, xcd=1700.0), _sample(0.95, xcd=1700.0),
         _sample(1.9, xcd=1650.0)]
    assert [x[0] for x in bench.refreshes(s)] == [0.0, 0.9, 1.9]


def test_clock_window_selects_the_window_and_averages():
    s = [_sample(0.9, xcd=2400.0, e_uj=0.0),
         _sample(1.0, xcd=1500.0, e_uj=1e6),
         _sample(1.01, xcd=1600.0, e_uj=1e6 + 14e6, power=1400),
         _sample(1.02, xcd=1700.0, e_uj=1e6 + 28e6, power=1420),
         _sample(1.5, xcd=100.0, e_uj=9e9)]
    r = bench.clock_window(s, 1.0, 1.02)
    assert r["samples"] == 3
    assert r["gfxclk_mhz_mean"] == pytest.approx(1600.0)
    assert r["gfxclk_mhz_min"] == 1500.0 and r["gfxclk_mhz_max"] == 1700.0
    assert r["socket_power_w_mean"] == pytest.approx((1380 + 1400 + 1420) / 3)
    # 28 J over 20 ms = 1.4 kW
    assert r["energy_power_w"] == pytest.approx(1400.0)
    assert r["throttle_status_any"] is False


def test_clock_window_falls_back_to_the_current_clock_and_skips_missing_values():
    s = [_sample(1.0, xcd=None, cur=1650, power=0xFFFF, e_uj=None),
         _sample(1.1, xcd=None, cur=0xFFFF, power=1200, e_uj=None)]
    r = bench.clock_window(s, 0.0, 2.0)
    assert r["gfxclk_mhz_mean"] == 1650
    assert r["socket_power_w_mean"] == 1200
    # a repeated table is one refresh
    assert bench.clock_window(s[:1] * 3, 0.0, 2.0)["samples"] == 1
    assert "energy_power_w" not in r
    assert bench.clock_window(s, 5.0, 6.0) == {"samples": 0, "window_ms": 1000.0}


def test_sampler_child_reports_a_missing_driver_without_failing():
    # on a host without the GPU driver the child answers with an error record
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--clock-sampler"],
                       input="\nstop\n", capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    import json
    d = json.loads(r.stdout.strip().splitlines()[-1])
    assert d["samples"] == [] or isinstance(d["samples"], list)
    if not d["samples"]:
        assert d["error"]


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
