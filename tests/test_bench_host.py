"""Host logic of bench.py, on the CPU: the one-GPU rule, the 70 %-of-peak bars
of the graded points, and the counter-measured traffic, which is reported only
while the decode kernel's source is the one the counters were taken on."""

import pytest

import bench


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().err


def test_world_size_above_one_is_refused(monkeypatch, capsys):
    monkeypatch.setenv("WORLD_SIZE", "2")
    assert bench.main([]) == 2
    assert "one GPU only" in capsys.readouterr().err


def test_bars_are_seventy_percent_of_peak():
    # the long-context step (1 073 938 432 bytes) and the MHA kv 4096 call:
    # 191.8 us and 6.0 us at 70 % of 8 TB/s
    assert bench.bar_us(1073938432) == pytest.approx(191.775, abs=1e-3)
    assert bench.bar_us(33562624) == pytest.approx(5.993, abs=1e-3)
    assert bench.bar_us(8_000_000, frac=1.0) == pytest.approx(1.0)


def test_graded_points_rows():
    per_kv = [{"kv_len": 1024, "bytes": 8396800, "call_us": 6.8},
              {"kv_len": 4096, "bytes": 33562624, "call_us": 10.4},
              {"kv_len": 8192, "bytes": 67117056, "call_us": 15.3}]
    minicpm = {"lockstep_p4095": {"bytes": 67174400, "us": 16.6},
               "lockstep_p8191": {"bytes": 134283264, "us": 26.1},
               "ragged": {"draws_mean_len_ge_4096": 0}}
    floor = [{"bytes": 33562624, "us": 6.7}, {"bytes": 1073938432, "us": 150.0}]
    rows = bench.graded_points(161.0, 1073938432, per_kv, minicpm, floor)
    names = [r["point"] for r in rows]
    assert len(rows) == 5 and not any("1024" in n for n in names)      # kv_len >= 4096 only
    assert not any("ragged" in n for n in names)                        # no qualifying draw
    lc = rows[-1]
    assert lc["meets_bar"] and lc["read_floor_us"] == 150.0
    assert lc["frac_of_peak"] == pytest.approx(1073938432 / 161.0 / 8e6, abs=1e-4)
    mha = rows[0]
    assert not mha["meets_bar"] and mha["read_floor_us"] == 6.7 and mha["bar_us"] == 5.99
    assert rows[1]["read_floor_us"] is None                             # no floor at that size


def test_traffic_only_for_the_profiled_kernel_source(tmp_path, monkeypatch):
    # the committed summary was taken on the committed kernel: its figure is
    # reported, reads plus writes of one 1.07 GB launch
    assert bench.pmc_traffic() == pytest.approx(1074724299.0)
    changed = tmp_path / "ada_kernels.hip"
    changed.write_bytes(bench.KERNEL_SOURCE.read_bytes() + b"\n// edited\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCE", changed)
    assert bench.pmc_traffic() is None
    monkeypatch.setattr(bench, "PMC_SUMMARY", tmp_path / "missing.md")
    assert bench.pmc_traffic() is None
