"""bench.py end to end on the GPU: one short run of the headline workload, in this process, and
the one JSON line it prints checked against the fields its consumers read."""
import json

import pytest

import bench

pytestmark = pytest.mark.gpu


def test_bench_prints_one_json_line_with_roofline_and_oracle_baseline(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--steps", "3", "--warmup", "1", "--cpu-seconds", "0.05",
                                     "--cpu-single-seconds", "0.05", "--cold", "2"])
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
    launch = r["launch_us"]
    assert launch["p10"] <= launch["median"] <= launch["p90"] and "10 further regions" in launch["spread_of"]
    assert roof["achieved"] == pytest.approx(r["config"]["algorithmic_bytes_per_step"] / launch["mean"] / 1e3, rel=1e-3)
    # the streaming ceiling over the same bytes, both walk orders, and the scan's share of it
    ceil = r["ceiling"]
    assert ceil["contiguous"]["rows"] == 1 and ceil["scan_order"]["rows"] == 32
    assert r["ceiling_gbs"] == ceil["contiguous"]["gbs"] > 0
    assert r["frac_of_ceiling"] == pytest.approx(roof["achieved"] / r["ceiling_gbs"], abs=1e-3)
    # the same stream in the plan's own tile walk (8-lane slabs, 1 wave, 8 rows per lane)
    tw = ceil["tile_walk"]
    assert (tw["lanes"], tw["waves"], tw["steps_per_lane"]) == (8, 1, 8) and tw["gbs"] > 0
    assert tw["frac_scan"] == pytest.approx(roof["achieved"] / tw["gbs"], abs=1e-3)
    single = r["single_launch_us"]
    assert single["cold"]["n"] == 2 and single["warm"]["n"] == 2 and single["cold"]["mean"] > 0
    cpu = r["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["unit"] == "GB/s" and cpu["value"] > 0 and cpu["cores"] >= 1
    assert cpu["host_cores"] >= cpu["cores"] and cpu["cpu_model"]
    assert cpu["single_thread"]["value"] > 0
    assert isinstance(cpu["sample"], str) and cpu["sample"]
    # the oracle's answer for the GPU's last output, within the parity bar
    assert cpu["gpu_check_max_bar_ratio"] <= 1.0


@pytest.mark.parametrize("extra,workload", [(["--workload", "tiny", "--no-cpu-baseline"], "tiny"),
                                            (["--dtype", "bf16", "--reverse", "--state", "--no-cpu-baseline"],
                                             "pages_shape"),
                                            (["--dtype", "bf16", "--cpu-seconds", "0.05",
                                              "--cpu-single-seconds", "0"], "pages_shape"),
                                            (["--workload", "long_sequence", "--reverse", "--a-ahead", "--state",
                                              "--cpu-seconds", "0.05", "--cpu-single-seconds", "0"],
                                             "long_sequence")],
                         ids=["tiny", "bf16_reverse_state", "bf16_checked", "decays_ahead_checked"])
def test_bench_other_workloads_and_forms(monkeypatch, capsys, extra, workload):
    monkeypatch.setattr("sys.argv", ["bench.py", "--steps", "3", "--warmup", "1", *extra])
    print(f"bench.main: {' '.join(extra)}", flush=True)
    bench.main()
    lines = [line for line in capsys.readouterr().out.splitlines() if line.startswith("{")]
    assert len(lines) == 1
    r = json.loads(lines[0])
    assert r["config"]["workload"].startswith(workload) and r["value"] > 0
    assert r["roofline"]["bound"] == "hbm" and r["roofline"]["achieved"] > 0
    # a counter record applies to forward scans without states of the same workload and storage
    forward = "--reverse" not in extra and "--state" not in extra
    dtype = r["config"]["storage"]
    assert r["roofline"]["traffic"] == (bench.measured_traffic(workload, dtype) if forward else None)
    if "bf16" in extra:
        assert r["config"]["storage"] == "bf16" and "bf16 storage" in r["config"]["workload"]
    if "--a-ahead" in extra:
        assert r["config"]["a_ahead"] is True and "decays one step ahead" in r["config"]["workload"]
    if "--no-cpu-baseline" in extra:
        assert r["cpu_baseline"] is None
    else:
        # the output checked against the oracle at the storage type's bar (for the decays one step
        # ahead: the oracle's reverse scan over a shifted copy of a, from the same initial state)
        assert r["cpu_baseline"]["gpu_check_max_bar_ratio"] <= 1.0 and "single_thread" not in r["cpu_baseline"]


def test_stream_rows_mode(monkeypatch, capsys):
    """--stream-rows times only the read-2-write-1 stream, once per row count, and prints one JSON
    line: contiguous (R = 1) and the scan's 32-row order of the headline buffers."""
    monkeypatch.setattr("sys.argv", ["bench.py", "--steps", "1", "--warmup", "1", "--stream-rows", "1,32"])
    print("bench.main: --stream-rows 1,32", flush=True)
    bench.main()
    lines = [line for line in capsys.readouterr().out.splitlines() if line.startswith("{")]
    assert len(lines) == 1
    r = json.loads(lines[0])
    assert r["kind"] == "stream_rows" and r["workload"] == "pages_shape"
    assert r["bytes_per_launch"] == 12 * 32 * 4096 * 256
    assert sorted(r["rows"]) == ["1", "32"]
    for key, rec in r["rows"].items():
        assert rec["rows"] == int(key) and rec["us"] > 0
        assert rec["gbs"] == pytest.approx(r["bytes_per_launch"] / rec["us"] / 1e3, rel=1e-3)
