"""Host logic of bench.py (no GPU): the HBM traffic derived from rocprofv3 counter files, and when a
stored traffic record applies."""
import csv
import json

import pytest

import bench

HEADER = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
SCAN = "void linrec::scan_tiles<float, 4, 8, 2>(float const*, float const*, float*, linrec::Geometry, ...)"
COPY = "__amd_rocclr_copyBuffer"


def write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HEADER)
        w.writerows(rows)
    return path


def test_counters_by_kernel_keeps_scan_and_copy_rows_in_bytes(tmp_path):
    path = write_csv(tmp_path / "c.csv", [
        [1, SCAN, "FETCH_SIZE", 100.0],
        [2, SCAN, "WRITE_SIZE", 7.0],                   # another counter: ignored
        [3, COPY, "FETCH_SIZE", 262144.0],
        [4, "some_other_kernel", "FETCH_SIZE", 5.0],    # another kernel: ignored
        [5, SCAN, "FETCH_SIZE", 300.0],
        [6, "void linrec::scan_one<float, 4, 4, 15>(float const*, ...)", "FETCH_SIZE", 50.0],
        [7, "void linrec::scan_relay<float, 4, 8, 1>(float const*, ...)", "FETCH_SIZE", 60.0],
    ])
    got = bench.counters_by_kernel(path, "FETCH_SIZE")
    assert got == {"scan": [100.0 * 1024, 300.0 * 1024, 50.0 * 1024, 60.0 * 1024], "copy": [262144.0 * 1024]}


def test_traffic_file_is_named_for_the_planned_kernel():
    assert bench.traffic_file("pages_shape").name == "traffic_scan_relay_pages_shape.json"
    assert bench.traffic_file("wide_channels").name == "traffic_scan_tiles_wide_channels.json"
    assert bench.traffic_file("long_sequence").name == "traffic_scan_one_long_sequence.json"
    assert bench.traffic_file("pages_shape", "bf16").name == "traffic_scan_one_pages_shape_bf16.json"
    assert bench.traffic_file("near_unit_resets", "f16").name == "traffic_scan_tiles_near_unit_resets_f16.json"


def test_current_plan_of_fp32_matches_the_plain_entry_point():
    from linear_recurrence_scan_linrec_amd import linrec as lr

    for name, w in bench.li.WORKLOADS.items():
        assert bench.current_plan(name) == lr.linrec_scan_plan(w.B, w.L, w.D), name


def test_traffic_record_scales_by_the_calibration_copy():
    # a 512 MiB copy reads as 256 MiB (FETCH_SIZE counts half) and writes as 512 MiB
    fetch = {"scan": [131072.0 * 1024, 131074.0 * 1024], "copy": [262144.0 * 1024] * 3}
    write = {"scan": [131072.0 * 1024] * 2, "copy": [524288.0 * 1024] * 3}
    rec = bench.traffic_record(fetch, write, "pages_shape")
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["read_bytes_per_launch"] == 2 * 131073 * 1024
    assert rec["written_bytes_per_launch"] == 131072 * 1024
    assert rec["hbm_bytes_per_launch"] == rec["read_bytes_per_launch"] + rec["written_bytes_per_launch"]
    assert rec["algorithmic_bytes_per_launch"] == 12 * 32 * 4096 * 256
    assert rec["scan_dispatches"] == [2, 2] and rec["copy_dispatches"] == [3, 3]
    assert rec["kernel_source_sha256"] == bench.kernel_source_hash()
    assert rec["storage"] == "f32"
    rec16 = bench.traffic_record(fetch, write, "pages_shape", "bf16")
    assert rec16["algorithmic_bytes_per_launch"] == 6 * 32 * 4096 * 256 and rec16["storage"] == "bf16"
    assert rec16["plan"] == bench.current_plan("pages_shape", "bf16")


def test_traffic_record_needs_both_kernels():
    with pytest.raises(SystemExit):
        bench.traffic_record({"scan": [1.0]}, {"scan": [1.0], "copy": [1.0]}, "pages_shape")


def test_kernel_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = tmp_path / "k.hpp"
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [src])
    src.write_text("int f(int x) { return x + 1; }  // one\n")
    h1 = bench.kernel_source_hash()
    src.write_text("/* header */\nint f(int x)   {\n  return x + 1;   // two\n}\n")
    assert bench.kernel_source_hash() == h1
    src.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_source_hash() != h1


def test_measured_traffic_applies_only_to_the_same_kernel_plan_and_workload(tmp_path, monkeypatch):
    record = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_file", lambda workload, dtype="f32": record)
    rec = {"workload": "pages_shape", "kernel_source_sha256": bench.kernel_source_hash(),
           "plan": bench.current_plan("pages_shape"), "hbm_bytes_per_launch": 403000000}
    record.write_text(json.dumps(rec))
    assert bench.measured_traffic("pages_shape") == 403000000
    record.write_text(json.dumps(dict(rec, kernel_source_sha256="0" * 64)))
    assert bench.measured_traffic("pages_shape") is None
    record.write_text(json.dumps(dict(rec, plan=dict(rec["plan"], waves=99))))
    assert bench.measured_traffic("pages_shape") is None
    record.write_text(json.dumps(rec))
    assert bench.measured_traffic("wide_channels") is None
    assert bench.measured_traffic("pages_shape", "bf16") is None     # a record of fp32 storage


def test_more_than_one_gpu_exits_with_a_message_before_touching_a_device(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err
