"""The measurement arithmetic of bench.py on the CPU: the algorithmic bytes
the roofline divides by, and the HBM traffic record built from two
rocprofv3 counter passes (calibration against the 1 GiB copy, the decode
and merge kernels summed, the source hash that retires a stale record)."""

import csv
import json

import bench


def test_algorithmic_bytes_by_hand():
    # two sequences of 17 and 0 tokens, 2 heads x 64: K and V of 17 tokens,
    # q in and out for both, two table entries and a length for the first,
    # a length for the second
    kv, total = bench.algorithmic_bytes([17, 0], 2, 64)
    assert kv == 17 * 2 * (2 * 64 * 2)
    assert total == kv + 2 * (2 * 64 * 2) * 2 + (2 * 4 + 4) + 4


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_record_calibrates_and_sums(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    dec = "void pkv::pa_decode_flat_kernel<128, 2, false, true>(pkv::FlatArgs)"
    mrg = "void pkv::pa_decode_flat_merge_kernel<128>(pkv::FlatArgs)"
    copy = "__amd_rocclr_copyBuffer"
    # FETCH_SIZE reads half of a 1 GiB copy (factor 2); a small input copy
    # must not enter the calibration
    _counter_csv(tmp_path / "fetch.csv", "FETCH_SIZE",
                 [(copy, 524288.0), (copy, 524288.0), (copy, 3.0),
                  (dec, 1000.0), (dec, 1002.0), (mrg, 10.0), (mrg, 10.0)])
    _counter_csv(tmp_path / "write.csv", "WRITE_SIZE",
                 [(copy, 1048576.0), (dec, 3.0), (mrg, 7.0)])
    bench.write_traffic_record(str(tmp_path / "fetch.csv"), str(tmp_path / "write.csv"))
    rec = json.load(open(tmp_path / "traffic.json"))
    assert rec["fetch_size_factor"] == 2.0 and rec["write_size_factor"] == 1.0
    assert rec["read_bytes"] == (1001 + 10) * 1024 * 2
    assert rec["write_bytes"] == (3 + 7) * 1024
    assert rec["pa_decode_hbm_bytes_per_call"] == rec["read_bytes"] + rec["write_bytes"]
    assert rec["kernel_source_sha256"] == bench.kernel_source_sha256()
    assert bench.measured_traffic() == rec["pa_decode_hbm_bytes_per_call"]
    # a record taken on other sources is not reported
    rec["kernel_source_sha256"] = "0" * 64
    json.dump(rec, open(tmp_path / "traffic.json", "w"))
    assert bench.measured_traffic() is None

