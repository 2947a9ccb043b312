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



def test_full_step_bytes_match_the_pages_per_token_figure():
    """The full decode step (32 layers x 200 sequences x 2048 tokens, 32
    heads x 128, fp16) moves K and V of 200 x 2048 tokens through every
    layer: the bench's per-layer K/V bytes summed over the 32 layers equal
    200 x 2048 x 524,288 B = 214,748,364,800 B, where 524,288 B (512 KiB)
    is the per-token cache size of "Atención paginada en modelos de lenguaje
    grandes (LLM)" (7minutos.es, bytes-per-token part: 2 (K and V) x 32
    layers x 32 heads x 128 dims x 2 bytes)."""
    import json
    import os

    import workloads as wl
    from paged_kv_cache_03_amd import kv_bytes_per_token

    golden = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                         "pages_worked_examples.json")))
    per_token = golden["bytes_per_token"]["bytes"]
    c = wl.full_step()
    assert c.num_layers == 32 and len(c.context_lens) == 200
    total = sum(bench.algorithmic_bytes(c.context_lens, c.num_heads, c.head_dim)[0]
                for _ in range(c.num_layers))
    assert kv_bytes_per_token(32, 32, 128) == per_token == 524288
    assert total == 200 * 2048 * kv_bytes_per_token(32, 32, 128) == 214_748_364_800


def _host_run(case, **extra):
    import torch
    return bench.Run(case=case, kp=torch.from_numpy(case.k_pool), vp=torch.from_numpy(case.v_pool),
                     extra=extra.pop("extra", {}), **extra)


def test_cpu_baseline_runs_the_oracle_over_a_worker_pool():
    """The CPU-baseline leg end to end on the host: the sample is written
    out, a child process times the oracle serially (single core) and over a
    pool of forked workers, for a decode, a grouped decode and a prefill
    sample; the record names the core count and both rates."""
    import torch

    import workloads as wl
    cases = [
        (_host_run(wl.gpt_batch(12, seed=1, append=True, num_blocks=1024, heads=4, head_dim=64)),
         "GB/s"),
        (_host_run(wl.shared_prefix(batch=6, seed=7, prefix_tokens=40, suffix_max=50, heads=4,
                                    head_dim=64), extra={"decode": "pa_decode_grouped"}), "GB/s"),
        (_host_run(wl.prefill(5, seed=3, heads=4, head_dim=64), prefill={"rows": 0},
                   chunked=False), "tokens/s"),
    ]
    for run, unit in cases:
        rec = bench.cpu_baseline(run, torch)
        assert rec["kind"] == "oracle" and rec["unit"] == unit
        assert rec["cores"] == bench.cpu_workers() >= 1
        assert rec["value"] > 0 and rec["single_core"]["value"] > 0
        assert rec["single_core"]["unit"] == unit
        assert "worker processes" in rec["sample"]
