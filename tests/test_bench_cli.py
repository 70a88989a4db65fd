"""bench.py's command-line contract: on the CPU, that it measures one GPU only
and refuses to run without one rather than falling back; on a GPU, the fields
of the JSON line it prints."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    res = run("--gpus", "2")
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_help_lists_the_contract_flags():
    res = run("--help")
    assert res.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--repeats", "--workload", "--b-layout", "--clock-seconds"):
        assert flag in res.stdout


@pytest.mark.gpu
def test_bench_prints_the_contract_line():
    # A short run on the 256^3 workload: one JSON line with the contract's fields;
    # the timed region is K back-to-back launches, so the kernel's average launch
    # duration over it gives roofline.achieved == value.
    res = run("--workload", "small_256", "--steps", "5", "--warmup", "5", "--repeats", "3", "--no-cpu-baseline",
              "--no-secondary", "--clock-seconds", "0")
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [l for l in res.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    j = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in j, key
    assert (j["n_gpus"], j["steps"], j["warmup"], j["unit"], j["dtype"], j["data"]) == (1, 5, 5, "TFLOP/s", "fp16",
                                                                                        "synthetic")
    assert j["config"]["workload"] == "small_256" and j["value"] > 0 and j["higher_is_better"] is True
    r = j["roofline"]
    assert (r["bound"], r["unit"], r["peak"]) == ("mfma", "TFLOP/s", 2500.0)
    assert r["achieved"] == j["value"] and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    # the median of the timed regions, each of exactly `steps` launches
    assert j["repeats"] == 3 and len(j["region_ms_per_step"]) == 3
    assert j["ms_per_step"] == sorted(j["region_ms_per_step"])[1]
    for side in ("first_timed_region", "last_timed_region"):
        assert set(j["clocks"][side]) == {"sclk_mhz", "mclk_mhz", "power_w"}


def test_zero_repeats_are_refused():
    res = run("--repeats", "0")
    assert res.returncode == 2


def _fake_sysfs(tmp_path, sclk_lines, power_uw, cap_uw):
    d = tmp_path / "card0" / "device"
    (d / "hwmon" / "hwmon3").mkdir(parents=True)
    (d / "vendor").write_text("0x1002\n")
    (d / "pp_dpm_sclk").write_text(sclk_lines)
    (d / "pp_dpm_mclk").write_text("0: 2000Mhz *\n")
    (d / "hwmon" / "hwmon3" / "power1_input").write_text(f"{power_uw}\n")
    (d / "hwmon" / "hwmon3" / "power1_cap").write_text(f"{cap_uw}\n")
    return str(d)


def test_clock_and_power_readers_parse_the_driver_files(tmp_path, monkeypatch):
    # The formats the amdgpu driver uses on these boards: the active shader-clock level is marked
    # with '*' (under load the middle level carries the live frequency, idle shows the sleep level).
    import bench
    d = _fake_sysfs(tmp_path, "S: 100Mhz\n0: 500Mhz\n1: 1608Mhz *\n2: 2400Mhz\n", 1353000000, 1400000000)
    monkeypatch.setattr(bench, "_SYSFS", d)
    assert bench.read_clocks() == {"sclk_mhz": 1608, "mclk_mhz": 2000, "power_w": 1353.0}
    assert bench.read_power_cap() == 1400.0
    ctx = bench.power_clock_context(1254.95, 2500.0, {"sclk_mhz": {"median": 1555}, "power_w": {"median": 1400.0}})
    assert ctx["peak_at_sustained_sclk"] == round(2500.0 * 1555 / 2400, 1)
    assert abs(ctx["frac_of_peak_at_sustained_sclk"] - 1254.95 / (2500.0 * 1555 / 2400)) < 1e-4
    assert (ctx["sustained_power_w"], ctx["power_cap_w"]) == (1400.0, 1400.0)


def test_clock_readers_report_unavailable_without_a_gpu(monkeypatch):
    import bench
    monkeypatch.setattr(bench, "_SYSFS", "")
    assert bench.read_clocks() == {"sclk_mhz": "unavailable", "mclk_mhz": "unavailable", "power_w": "unavailable"}
    assert bench.read_power_cap() == "unavailable"
    assert bench.power_clock_context(1.0, 2500.0, None)["sustained_sclk_mhz"] == "unavailable"


def test_sysfs_card_is_chosen_by_pci_address(tmp_path):
    # Two AMD cards whose device links point at their PCI directories: the one whose address is the
    # measured GPU's is chosen; an unknown or missing address falls back to the first card.
    import bench
    drm, pci = tmp_path / "drm", tmp_path / "pci"
    for card, addr in (("card0", "0000:03:00.0"), ("card1", "0000:83:00.0")):
        dev = pci / addr
        dev.mkdir(parents=True)
        (dev / "vendor").write_text("0x1002\n")
        (dev / "pp_dpm_sclk").write_text("0: 2400Mhz *\n")
        (drm / card).mkdir(parents=True)
        os.symlink(dev, drm / card / "device")
    (drm / "card2").mkdir()                       # a card without a device link is skipped
    chosen = bench._gpu_sysfs_dir("0000:83:00.0", root=str(drm))
    assert os.path.realpath(chosen) == str(pci / "0000:83:00.0")
    assert os.path.realpath(bench._gpu_sysfs_dir("0000:03:00.0", root=str(drm))) == str(pci / "0000:03:00.0")
    assert os.path.realpath(bench._gpu_sysfs_dir("0000:99:00.0", root=str(drm))) == str(pci / "0000:03:00.0")
    assert os.path.realpath(bench._gpu_sysfs_dir(None, root=str(drm))) == str(pci / "0000:03:00.0")
    assert bench._gpu_sysfs_dir(None, root=str(tmp_path / "none")) is None
