"""bench.py end to end on the GPU: one short run of the headline workload, in this process, and
the one JSON line it prints checked against the fields its consumers read."""
import json

import pytest

import bench

pytestmark = pytest.mark.gpu


def test_bench_prints_one_json_line_with_roofline_and_oracle_baseline(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--steps", "3", "--warmup", "1", "--cpu-seconds", "0.05"])
    print("bench.main: pages_shape, 3 steps", flush=True)
    bench.main()
    lines = [line for line in capsys.readouterr().out.splitlines() if line.startswith("{")]
    assert len(lines) == 1
    r = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in r, key
    assert r["metric"] == bench.METRIC and r["unit"] == "GB/s" and r["value"] > 0
    assert (r["n_gpus"], r["steps"], r["warmup"]) == (1, 3, 1)
    assert r["higher_is_better"] is True and r["data"] == "synthetic" and r["dtype"] == "f32"
    assert r["config"]["workload"].startswith("pages_shape")
    assert (r["config"]["B"], r["config"]["L"], r["config"]["D"]) == (32, 4096, 256)
    roof = r["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == bench.PEAK_HBM_GBS
    assert 0 < roof["achieved"] <= roof["peak"]
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-4)
    assert roof["traffic"] == bench.measured_traffic("pages_shape")
    cpu = r["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["unit"] == "GB/s" and cpu["value"] > 0 and cpu["cores"] >= 1
    assert isinstance(cpu["sample"], str) and cpu["sample"]
    # the oracle's answer for the GPU's last output, within the parity bar
    assert cpu["gpu_check_max_ratio"] <= 1e-4


@pytest.mark.parametrize("extra,workload", [(["--workload", "tiny"], "tiny"),
                                            (["--dtype", "bf16", "--reverse", "--state"], "pages_shape")],
                         ids=["tiny", "bf16_reverse_state"])
def test_bench_other_workloads_and_forms(monkeypatch, capsys, extra, workload):
    monkeypatch.setattr("sys.argv", ["bench.py", "--steps", "3", "--warmup", "1", "--no-cpu-baseline", *extra])
    print(f"bench.main: {' '.join(extra)}", flush=True)
    bench.main()
    lines = [line for line in capsys.readouterr().out.splitlines() if line.startswith("{")]
    assert len(lines) == 1
    r = json.loads(lines[0])
    assert r["config"]["workload"].startswith(workload) and r["value"] > 0 and r["cpu_baseline"] is None
    assert r["roofline"]["bound"] == "hbm" and r["roofline"]["achieved"] > 0
    plain = workload != "pages_shape"   # the second case runs through linrec_scan_ex
    assert r["roofline"]["traffic"] == (bench.measured_traffic(workload) if plain else None)
