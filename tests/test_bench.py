"""bench.py: host logic on the CPU, and the one-line JSON contract on the GPU."""
import json
import math
import time

import pytest

import bench
import datagen


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_bad_settle_is_refused(capsys):
    assert bench.main(["--settle", "-1"]) == 2
    assert "--settle" in capsys.readouterr().err


def test_workload_flops_and_bytes():
    w = datagen.WORKLOADS[3]
    assert w.flops == 4 * 2 * 16 * 4096 * 4096 * 128
    # Q, K, V read and O written once (bf16), lse written once (fp32)
    assert bench.algorithmic_bytes(w) == 4 * 2 * 16 * 4096 * 128 * 2 + 4 * 2 * 16 * 4096


def test_traffic_only_for_the_profiled_kernel_source(tmp_path, monkeypatch):
    w = datagen.WORKLOADS[3]
    rec = {"kernel_sha256_16": bench.kernel_source_hash(),
           "workloads": {"3": {"hbm_bytes_per_launch": 123}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_for(w) == 123
    assert bench.traffic_for(datagen.WORKLOADS[4]) is None      # not profiled
    rec["kernel_sha256_16"] = "0" * 16                            # source changed since
    f.write_text(json.dumps(rec))
    assert bench.traffic_for(w) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_for(w) is None


def test_kernel_source_hash_is_stable():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()


def test_cpu_baseline_times_the_oracle():
    w = datagen.WORKLOADS[1]
    q, k, v = datagen.workload_inputs(1)
    cb = bench.cpu_baseline(w, q, k, v, budget_s=0.2)
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert "of 128 query rows" in cb["sample"]


@pytest.mark.gpu
@pytest.mark.parametrize("extra", [[], ["--causal"], ["--backward"], ["--splitkv", "2"]])
def test_bench_json_line(extra, capsys):
    assert bench.main(["--workload", "2", "--steps", "3", "--warmup", "1",
                       "--no-cpu-baseline", *extra]) == 0
    lines = [x for x in capsys.readouterr().out.splitlines() if x.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    # an explicit warmup count comes after the default 0.25 s settle phase
    assert d["settle"]["seconds"] == 0.25 and d["settle"]["launches"] >= 20
    assert d["unit"] == "TFLOP/s" and d["higher_is_better"] is True
    assert d["config"]["workload"] == datagen.WORKLOADS[2].name
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["peak"] == 2500.0 and r["unit"] == "TFLOP/s"
    assert 0.0 < r["achieved"] < r["peak"]
    assert math.isclose(r["frac"], r["achieved"] / r["peak"], rel_tol=1e-3, abs_tol=1e-4)
    assert d["value"] > 0 and d["ms_per_step"] > 0
    c = d["clock"]  # None where the driver's sysfs files are not readable
    if c is not None:
        assert c["samples"] >= 1
        if c["window_s"] < 0.25:  # a few launches: nothing measured is reported
            assert c["sclk_mhz"] is None and c["power_w"] is None and c["frac_at_clock"] is None
        else:
            assert 0 < c["sclk_mhz"] <= 3000
        if c["frac_at_clock"] is not None:
            assert math.isclose(c["frac_at_clock"], r["achieved"] / c["peak_at_clock"],
                                rel_tol=1e-2)
    if "--backward" in extra:
        assert d["metric"].startswith("attention bwd")


def test_decode_bytes_and_splits():
    w = datagen.DECODE
    assert (w["B"], w["H"], w["N"], w["Nk"], w["d"], w["dtype"]) == (1, 32, 1, 65536, 128, "bf16")
    # K and V read once (bf16), Q read and O written once, lse written once (fp32)
    assert bench.decode_bytes(w) == 2 * 32 * 65536 * 128 * 2 + 2 * 32 * 128 * 2 + 4 * 32
    assert bench.decode_splits(w) == 16                      # 32 heads x 16 = 512 blocks
    assert bench.decode_splits(dict(w, B=64)) == 1           # 2048 heads fill the GPU alone
    assert bench.decode_splits(dict(w, H=1, Nk=300)) == 5    # at most one split per key tile
    assert bench.decode_splits(dict(w, H=1)) == 64


def test_cpu_baseline_decode_times_the_oracle():
    w = dict(datagen.DECODE, Nk=4096, H=4)
    q, k, v = datagen.make_qkv_kv(w["B"], w["H"], w["N"], w["Nk"], w["d"], w["dtype"], 1)
    cb = bench.cpu_baseline_decode(w, q, k, v, 0.088, budget_s=0.05)
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s" and cb["value"] > 0
    assert "of 4 heads" in cb["sample"]


@pytest.mark.gpu
def test_bench_decode_json_line(capsys):
    assert bench.main(["--decode", "--steps", "3", "--warmup", "1", "--no-cpu-baseline"]) == 0
    d = json.loads([x for x in capsys.readouterr().out.splitlines() if x.strip()][-1])
    assert d["unit"] == "GB/s" and d["steps"] == 3 and d["config"]["Nk"] == 65536
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and 0.0 < r["achieved"] < 8000.0
    assert math.isclose(r["frac"], r["achieved"] / r["peak"], rel_tol=1e-3, abs_tol=1e-4)


def test_parse_sclk_reads_the_current_level():
    assert bench.parse_sclk("0: 500Mhz\n1: 1650Mhz *\n2: 2400Mhz\n") == 1650.0
    assert bench.parse_sclk("S: 94Mhz *\n0: 500Mhz\n1: 2400Mhz\n") == 94.0
    assert bench.parse_sclk("0: 500Mhz\n1: 2400Mhz\n") is None


def test_clock_sampler_summary(tmp_path):
    (tmp_path / "pp_dpm_sclk").write_text("0: 500Mhz\n1: 1600Mhz *\n2: 2400Mhz\n")
    hw = tmp_path / "hwmon" / "hwmon0"
    hw.mkdir(parents=True)
    (hw / "power1_input").write_text("1290000000\n")
    (hw / "power1_cap").write_text("1400000000\n")
    with bench.ClockSampler(period_s=0.005, sysfs_dir=str(tmp_path)) as c:
        time.sleep(0.3)
    s = c.summary(achieved=1200.0, peak=2500.0)
    assert s["samples"] >= 2 and s["sclk_mhz"] == 1600.0 and s["window_s"] >= 0.25
    assert s["power_w"] == 1290.0 and s["power_cap_w"] == 1400.0
    assert math.isclose(s["peak_at_clock"], 2500.0 * 1600 / 2400, rel_tol=1e-3)
    assert math.isclose(s["frac_at_clock"], 1200.0 / (2500.0 * 1600 / 2400), rel_tol=1e-3)


def test_clock_sampler_without_sysfs_reports_nothing(tmp_path):
    with bench.ClockSampler(period_s=0.001, sysfs_dir=str(tmp_path)) as c:
        time.sleep(0.01)
    assert c.summary(1.0, 2.0) is None


def test_short_window_gives_no_clock_fraction(tmp_path):
    (tmp_path / "pp_dpm_sclk").write_text("1: 1100Mhz *\n")
    with bench.ClockSampler(period_s=0.001, sysfs_dir=str(tmp_path)) as c:
        time.sleep(0.02)
    s = c.summary(achieved=1200.0, peak=2500.0)
    assert s["samples"] >= 1 and s["window_s"] < 0.25
    for key in ("sclk_mhz", "sclk_mhz_min", "sclk_mhz_max", "power_w", "peak_at_clock",
                "frac_at_clock"):
        assert s[key] is None, key


def test_step_counts_are_checked(capsys):
    assert bench.main(["--steps", "0"]) == 2
    assert bench.main(["--warmup", "-1"]) == 2
    assert "--steps" in capsys.readouterr().err


@pytest.mark.gpu
def test_bench_default_counts_are_time_based(capsys):
    """Without --steps/--warmup: at least 200 warmup launches over >= 0.3 s,
    then at least 200 timed ones over about a second."""
    assert bench.main(["--workload", "2", "--no-cpu-baseline"]) == 0
    d = json.loads([x for x in capsys.readouterr().out.splitlines() if x.strip()][-1])
    assert d["warmup"] >= 200 and d["steps"] >= 200
    assert d["settle"] is None  # the automatic warmup is the settle phase itself
    assert d["steps"] * d["ms_per_step"] >= 500.0  # about 1 s of timed launches
    c = d["clock"]
    if c is not None:
        assert c["window_s"] >= 0.5 and c["frac_at_clock"] is not None
