"""Host-side parts of bench.py: the sysfs power and clock readers against a
synthetic sysfs tree and the one-GPU guard (CPU), and the readers on a GPU
host (gpu)."""
import os
import subprocess
import sys
import time

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_read_sclk_takes_the_marked_level(tmp_path):
    (tmp_path / "pp_dpm_sclk").write_text("0: 500Mhz\n1: 1834Mhz *\n2: 2400Mhz\n")
    assert bench._read_sclk(str(tmp_path)) == 1834.0
    (tmp_path / "pp_dpm_sclk").write_text("S: 95Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    assert bench._read_sclk(str(tmp_path)) == 95.0
    assert bench._read_sclk(str(tmp_path / "missing")) is None


def test_power_during_reads_the_sensor(tmp_path, monkeypatch):
    mon, dev = tmp_path / "hwmon0", tmp_path / "device"
    mon.mkdir()
    dev.mkdir()
    (mon / "power1_input").write_text("1398000000\n")        # microwatts
    (mon / "power1_cap").write_text("1400000000\n")
    (dev / "pp_dpm_sclk").write_text("0: 500Mhz\n1: 1835Mhz *\n")
    monkeypatch.setattr(bench, "_gpu_hwmon", lambda: (str(mon), str(dev)))
    monkeypatch.setattr(bench.torch.cuda, "synchronize", lambda *a, **k: None)
    calls = []

    def run():
        time.sleep(0.05)
        calls.append(1)
        return [16.25]

    p = bench.power_during(run, 0.6)
    assert p is not None and p["samples"] > 0
    assert p["board_w"] == 1398.0 and p["board_w_max"] == 1398.0 and p["cap_w"] == 1400.0
    assert p["sclk_mhz"] == 1835.0 and p["ms_per_launch_median"] == 16.25
    assert len(calls) >= 5 and p["seconds"] >= 0.6


def test_power_during_without_a_sensor(monkeypatch):
    monkeypatch.setattr(bench, "_gpu_hwmon", lambda: (None, None))
    assert bench.power_during(lambda: [1.0], 1.0) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr


@pytest.mark.gpu
def test_power_during_on_the_gpu():
    """On a GPU host the sensor of device 0 is found (where sysfs shows it)
    and reads a plausible board power and shader clock while a kernel runs."""
    if not bench.torch.cuda.is_available():
        pytest.skip("needs a GPU")
    x = bench.torch.empty(1 << 26, device="cuda")

    def run():
        for _ in range(20):
            x.neg_()
        bench.torch.cuda.synchronize()
        return [1.0]

    p = bench.power_during(run, 1.5)
    mon, _ = bench._gpu_hwmon()
    if mon is None:
        assert p is None
        return
    assert p is not None and p["samples"] > 0
    assert 50.0 < p["board_w"] <= (p["cap_w"] or 5000.0) * 1.1
    assert p["sclk_mhz"] is None or 50.0 <= p["sclk_mhz"] <= 3000.0
