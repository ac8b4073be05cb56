"""bench.py's clock sampler reads the driver's sysfs files correctly (CPU only:
a fake sysfs tree stands in for the card)."""
import os
import time

import bench


def _card(root, sclk_text, power_uw=None, cap_uw=None, name="card0"):
    dev = os.path.join(root, name, "device")
    os.makedirs(os.path.join(dev, "hwmon", "hwmon0"))
    with open(os.path.join(dev, "pp_dpm_sclk"), "w") as f:
        f.write(sclk_text)
    if power_uw is not None:
        with open(os.path.join(dev, "hwmon", "hwmon0", "power1_input"), "w") as f:
            f.write(f"{power_uw}\n")
    if cap_uw is not None:
        with open(os.path.join(dev, "hwmon", "hwmon0", "power1_cap"), "w") as f:
            f.write(f"{cap_uw}\n")


def test_sampler_reads_marked_level_and_power(tmp_path):
    _card(str(tmp_path), "S: 1830Mhz *\n0: 500Mhz\n1: 2400Mhz\n", 1234500000, 1400000000)
    with bench.ClockSampler(period=0.001, root=str(tmp_path)) as c:
        time.sleep(0.02)
    s = c.summary()
    assert s["sclk_mhz_median"] == 1830 and s["sclk_mhz_min"] == 1830 and s["samples"] >= 1
    assert s["power_w_median"] == 1234.5 and s["power_cap_w"] == 1400.0


def test_sampler_marked_dpm_level(tmp_path):
    _card(str(tmp_path), "0: 500Mhz\n1: 2400Mhz *\n")
    with bench.ClockSampler(period=0.001, root=str(tmp_path)) as c:
        time.sleep(0.01)
    s = c.summary()
    assert s["sclk_mhz_median"] == 2400 and "power_w_median" not in s


def test_sampler_absent_or_ambiguous(tmp_path):
    with bench.ClockSampler(root=str(tmp_path / "none")) as c:
        pass
    assert c.summary() is None
    _card(str(tmp_path), "S: 1830Mhz *\n", name="card0")
    _card(str(tmp_path), "S: 1900Mhz *\n", name="card1")
    with bench.ClockSampler(root=str(tmp_path)) as c:
        pass
    assert c.summary() is None
