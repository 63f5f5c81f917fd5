"""Host-only checks of bench.py's clock and power sampler against a fake sysfs
tree (the GPU machine exposes the same files under its PCI device directory)."""
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import bench  # noqa: E402


def _fake_device(tmp_path, with_power=True):
    dev = tmp_path / "dev"
    dev.mkdir()
    (dev / "pp_dpm_sclk").write_text("0: 500Mhz\n1: 1735Mhz *\n2: 2400Mhz\n")
    if with_power:
        hw = dev / "hwmon" / "hwmon3"
        hw.mkdir(parents=True)
        (hw / "power1_average").write_text("1270000000\n")  # microwatts
        (hw / "power1_cap").write_text("1400000000\n")
    return str(dev)


def test_sampler_reports_the_current_level_and_the_socket_power(tmp_path):
    src = _fake_device(tmp_path)
    with bench.ClockSampler(src) as s:
        time.sleep(0.02)
    out = s.summary()
    assert out["sclk_mhz_median"] == 1735 and out["sclk_mhz_min"] == 1735 and out["samples"] > 0
    assert out["power_w_median"] == 1270.0 and out["power_w_max"] == 1270.0
    assert out["power_cap_w"] == 1400.0


def test_sampler_without_power_files_reports_clocks_only(tmp_path):
    src = _fake_device(tmp_path, with_power=False)
    with bench.ClockSampler(src) as s:
        time.sleep(0.02)
    out = s.summary()
    assert out["sclk_mhz_median"] == 1735
    assert "power_w_median" not in out and "power_cap_w" not in out


def test_sampler_without_a_source_is_silent():
    with bench.ClockSampler(None) as s:
        pass
    assert s.summary() is None
