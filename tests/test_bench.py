"""bench.py: host logic on the CPU, and the one-line JSON contract on the GPU."""
import json
import math

import pytest

import bench
import datagen


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


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
    assert d["unit"] == "TFLOP/s" and d["higher_is_better"] is True
    assert d["config"]["workload"] == datagen.WORKLOADS[2].name
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["peak"] == 2500.0 and r["unit"] == "TFLOP/s"
    assert 0.0 < r["achieved"] < r["peak"]
    assert math.isclose(r["frac"], r["achieved"] / r["peak"], rel_tol=1e-3, abs_tol=1e-4)
    assert d["value"] > 0 and d["ms_per_step"] > 0
    if "--backward" in extra:
        assert d["metric"].startswith("attention bwd")
