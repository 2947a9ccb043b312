"""Throughput of the paged-decode hot path on one MI355X.

One step = one pass of the hot path over one batch: append one new token per
sequence into its slot (kv_append), then decode every sequence over its
whole context (pa_decode: decode kernel + merge kernel).  The workload is
one layer of a GPT-style model, batch 200, 32 heads x 128 dims, fp16,
16-token blocks, contexts = prompt U[32,256] + response geometric(mean 500)
capped at 2048, pool = blocks needed + 10% free, tables from a shuffled free
list (seed 2).  Inputs are resident in HBM before the timed region.

The default run then times the other workloads in the same process (batch
10, the shared prefix with the grouped decode, the 32-layer full step, the
4-beam full step, the prompt prefill and the chunked prefill) and adds a
summary of each (step time and rate, call time, roofline on its own bytes,
seq-layers/s, its own CPU baseline) under ``other_workloads``; ``--workload``
runs one of them alone, ``--no-extras`` skips them.

The CPU baseline is the float64 oracle on a bounded sample of each workload,
run by a child process that never touches the GPU, over a pool of up to 16
worker processes with one BLAS thread each, next to a single-core figure.

Prints one JSON line.  ``--gpus`` above 1 is refused: the library runs on
one GPU (there is no multi-GPU path).
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pa_decode_flat_batch200_hbm_traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--partition", type=int, default=0, help="partition tokens (0 = default)")
    ap.add_argument("--workload", default="batch200",
                    choices=["batch200", "batch10", "shared_prefix", "full_step", "beam_step",
                             "prefill_prompt", "prefill_chunked", "vattention"],
                    help="batch200 (default): the headline one-layer batch of 200")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="default workload only: skip timing the other workloads (batch 10, "
                         "shared prefix, full step, 4-beam step, both prefills) in the same run")
    ap.add_argument("--cpu-worker", metavar="DIR", help=argparse.SUPPRESS)
    ap.add_argument("--lds-probe", action="store_true",
                    help="only time the LDS read probe (one workgroup per CU, both read forms) "
                         "and print its rates as one JSON line")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain device copy of known size (counter calibration)")
    ap.add_argument("--decode", choices=["auto", "flat", "grouped"], default="auto",
                    help="decode entry point: pa_decode (flat strategy unless --partition) or "
                         "pa_decode_grouped (each shared block read once per group); auto = "
                         "grouped for the workloads whose tables share blocks")
    ap.add_argument("--vkv-chunk", type=int, default=2 << 20,
                    help="vattention workload: bytes of physical memory mapped at a time")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM-traffic record from two rocprofv3 counter_collection "
                         "CSVs (FETCH_SIZE pass, WRITE_SIZE pass; both runs with --copy-probe) "
                         "and exit; needs no GPU")
    ap.add_argument("--separate-append", action="store_true",
                    help="batch, full-step and prefill workloads: kv_append then pa_decode "
                         "or pa_prefill (two launches) instead of the fused pa_decode_append "
                         "or pa_prefill_append")
    ap.add_argument("--fused-append", action="store_true",
                    help="prefill_chunked: one pa_prefill_append call instead of kv_append "
                         "then pa_prefill")
    ap.add_argument("--no-hbm-probe", action="store_true",
                    help="skip the HBM read probes (achievable-bandwidth references)")
    ap.add_argument("--cold-reps", type=int, default=10,
                    help="one-layer workloads: calls timed after writing a 1 GiB scratch "
                         "buffer, which evicts the L2 and the 256 MB MALL (0 = skip)")
    return ap.parse_args(argv)


def default_args():
    return parse([])


# Workloads timed after the headline in a default run: (name, timed steps,
# warmup steps).  A full step is 32 layers, about 33 ms.
EXTRA_WORKLOADS = [("batch10", 50, 10), ("shared_prefix", 50, 10), ("full_step", 3, 1),
                   ("beam_step", 5, 2), ("prefill_prompt", 20, 5), ("prefill_chunked", 20, 5)]
ONE_LAYER = ("batch10", "shared_prefix", "prefill_prompt", "prefill_chunked")


def summarise(rec):
    """The fields of another workload's record that go into the headline
    line: its step time and rate, its call time, its roofline, seq-layers/s
    and its own CPU baseline."""
    keep = ("metric", "value", "unit", "ms_per_step", "steps", "warmup", "seq_layers_per_s",
            "pa_decode_us", "pa_decode_us_median", "pa_decode_kv_gbs", "pa_decode_pct_hbm_peak",
            "pa_decode_unique_kv_gbs", "pa_decode_us_cold_median", "pa_prefill_us",
            "pa_prefill_us_median", "pa_prefill_tflops", "pa_prefill_gbs",
            "pa_decode_us_back_to_back", "pa_prefill_us_back_to_back",
            "pa_prefill_us_cold_median", "decode", "groups", "layers", "query_rows")
    out = {"config": rec["config"]}
    out.update({k: rec[k] for k in keep if k in rec})
    out["roofline"] = {k: v for k, v in rec["roofline"].items() if k != "traffic"}
    if "cpu_baseline" in rec:
        out["cpu_baseline"] = rec["cpu_baseline"]
    return out


def algorithmic_bytes(lens, H, D):
    """Per decode launch: K and V of every context token, q in and out, the
    block-table entries read, the context length."""
    lens = [int(x) for x in lens]
    kv = sum(lens) * 2 * H * D * 2
    qo = len(lens) * H * D * 2 * 2
    tab = sum(4 * math.ceil(n / 16) + 4 for n in lens)
    return kv, kv + qo + tab


def lds_probe(torch, dev, rounds=4000):
    """LDS read rate per CU with pkv_lds_read_probe: one workgroup per CU of
    4, 8 or 16 waves, each wave reading 64 KiB of LDS `rounds` times in 16-byte
    row reads (form 0, 16 KiB per round) or in the prefill's transpose reads
    (form 1, 8 KiB per round).  Bytes per shader clock per CU from each
    workgroup's slowest wave (median over the CUs), the clock from the same
    cycles over the launch's event time."""
    import numpy as np
    from paged_kv_cache_03_amd.ops import lds_read_probe
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = {"rounds": rounds, "workgroups": cus}
    for form, per_round in ((0, 16 * 1024), (1, 8 * 1024)):
        for waves in (4, 8, 16):
            cyc = torch.zeros(cus * waves, dtype=torch.int64, device=dev)
            sink = torch.zeros(cus * waves, dtype=torch.int32, device=dev)
            lds_read_probe(cyc, sink, cus, waves, 10, form)
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            lds_read_probe(cyc, sink, cus, waves, rounds, form)
            e.record()
            torch.cuda.synchronize()
            us = s.elapsed_time(e) * 1e3
            wg = cyc.cpu().numpy().reshape(cus, waves).max(axis=1)
            bpc = waves * rounds * per_round / wg
            out[f"form{form}_waves{waves}"] = {
                "bytes_per_clock_per_cu": round(float(np.median(bpc)), 1),
                "min": round(float(bpc.min()), 1), "max": round(float(bpc.max()), 1),
                "instructions_per_clock_per_cu": round(float(np.median(bpc)) / (per_round / 16), 3),
                "us": round(us, 1), "clock_ghz": round(float(np.median(wg)) / us / 1e3, 3)}
            log(f"lds probe form {form} waves {waves}: {out[f'form{form}_waves{waves}']}")
    return out


def copy_probe(torch, dev, nbytes=1 << 30):
    """Achievable read + write rate of a plain device copy (as many bytes
    written as read: the mix of the prefill with its append fused in, which
    reads q and the new rows and writes out and the pools), the best over a
    few grid sizes of pkv_hbm_copy_probe, in GB/s of bytes read + written."""
    from paged_kv_cache_03_amd.ops import hbm_copy_probe
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    best = 0.0
    for w in (1024, 4096, 16384):
        for _ in range(2):
            hbm_copy_probe(src, dst, w)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(10):
            hbm_copy_probe(src, dst, w)
        e.record()
        torch.cuda.synchronize()
        best = max(best, 2 * nbytes / (s.elapsed_time(e) / 10 / 1e3) / 1e9)
    del src, dst
    return round(best, 1)


def hbm_probe(torch, dev, nbytes=2 << 30):
    """Achievable HBM read rates next to the 8 TB/s published peak: a plain
    linear read, and a gather of 4 KiB chunks in random order (the decode's
    pattern: one head's 16-token block, scattered over the pool), each the
    best over a few grid sizes."""
    import numpy as np
    from paged_kv_cache_03_amd.ops import hbm_gather_probe, hbm_read_probe
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    chunk = 4096
    perm = np.random.default_rng(0).permutation(nbytes // chunk).astype(np.int32)
    order = torch.from_numpy(perm).to(dev)

    def rate(call):
        for _ in range(2):
            call()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(10):
            call()
        e.record()
        torch.cuda.synchronize()
        return nbytes / (s.elapsed_time(e) / 10 / 1e3) / 1e9

    lin = max((rate(lambda: hbm_read_probe(buf, sink, w)), w) for w in (256, 512, 1024, 2048))
    gat = max((rate(lambda: hbm_gather_probe(buf, order, chunk, sink, w)), w) for w in (512, 1024))
    del buf, order
    return {"bytes": nbytes, "linear_gbs": round(lin[0], 1), "linear_workgroups": lin[1],
            "gather_4k_gbs": round(gat[0], 1), "gather_workgroups": gat[1]}


def kernel_source_sha256():
    """Hash of the sources the pa_decode call is built from (kernels, shared
    device code, launch plan), to tell whether stored counter figures still
    describe the code that runs."""
    import hashlib
    h = hashlib.sha256()
    for name in ("api.hip", "kernels.h", "pa_common.h", "pa_decode.hip", "pa_decode_flat.hip"):
        rel = os.path.join("paged_kv_cache_03_amd", "csrc", name)
        h.update(rel.encode())
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per pa_decode call from the committed rocprofv3 counter
    passes (FETCH_SIZE, WRITE_SIZE, calibrated against a 1 GiB copy), or None
    once the kernel sources differ from the ones they were taken on."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except OSError:
        return None
    if rec.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    return int(rec["pa_decode_hbm_bytes_per_call"])


def counter_kib_by_kernel(path, counter):
    """Values of ``counter`` (KiB per dispatch), listed by kernel name, from a
    rocprofv3 counter_collection CSV."""
    import csv
    vals = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter:
                vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return vals


def write_traffic_record(fetch_csv, write_csv, workload="batch200_seed2_pa_decode_append"):
    """HBM bytes per pa_decode call (decode + merge kernels) from the two
    counter passes, each scaled by what the same counter reads for the 1 GiB
    device copy of --copy-probe (bytes moved / counter bytes), stored with the
    hash of the kernel sources it describes."""
    n = 1 << 30
    rec = {"workload": workload, "kernel_source_sha256": kernel_source_sha256()}
    total = 0
    for which, path, counter in (("read", fetch_csv, "FETCH_SIZE"),
                                 ("write", write_csv, "WRITE_SIZE")):
        vals = counter_kib_by_kernel(path, counter)
        mean = lambda xs: sum(xs) / len(xs)
        # the 1 GiB copies, not the small host-to-device copies of the inputs
        copies = [v for k, xs in vals.items() if "copyBuffer" in k for v in xs]
        copies = [v for v in copies if v >= 0.5 * max(copies, default=0.0)]
        dec = [xs for k, xs in vals.items() if "pa_decode_flat_kernel" in k]
        mrg = [xs for k, xs in vals.items() if "pa_decode_flat_merge_kernel" in k]
        if not copies or len(dec) != 1 or len(mrg) != 1:
            raise SystemExit(f"{path}: expected the copy probe, one decode and one merge kernel")
        factor = n / (mean(copies) * 1024)
        b = int(round((mean(dec[0]) + mean(mrg[0])) * 1024 * factor))
        rec[f"{which}_bytes"] = b
        rec[f"{counter.lower()}_factor"] = round(factor, 4)
        total += b
    rec["pa_decode_hbm_bytes_per_call"] = total
    rec["source"] = "pa_decode_flat_batch200_hbm_counters.md"
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def _sample_pools(tables, kp, vp, torch):
    """The blocks a sample of table rows reads, copied to the host as compact
    pools, and the rows renumbered into them."""
    import numpy as np
    ids = np.unique(tables.reshape(-1))
    ids = ids[ids >= 0]
    remap = np.full(int(ids.max()) + 1 if ids.size else 1, -1, dtype=np.int32)
    remap[ids] = np.arange(len(ids), dtype=np.int32)
    idx = torch.from_numpy(ids.astype(np.int64)).to(kp.device)
    k_small = kp.index_select(0, idx).cpu().numpy()
    v_small = vp.index_select(0, idx).cpu().numpy()
    rows = np.where(tables >= 0, remap[np.maximum(tables, 0)], -1).astype(np.int32)
    return k_small, v_small, rows


# Host threads the CPU baseline may use: the cores this process may run on,
# at most 16 (the host share of one GPU).
CPU_WORKERS_MAX = 16


def cpu_workers():
    return max(1, min(len(os.sched_getaffinity(0)), CPU_WORKERS_MAX))


def cpu_sample(run, torch):
    """The oracle's inputs for a bounded sample of the workload, as host
    arrays: every sequence of a one-layer decode (whole groups for the
    grouped decode), layer 0 of a full step (the per-step figure is that
    layer's rate, an extrapolation to the step's layers), all prompts of the
    prompt prefill, the first 8 sequences of the chunked prefill."""
    import numpy as np

    import workloads as wl
    case = run.case
    q_all = case.q[0] if case.q.ndim == 4 else case.q
    prefill = getattr(run, "prefill", None) is not None
    grouped = run.extra.get("decode") == "pa_decode_grouped"
    meta = {"scale": float(case.scale), "heads": case.num_heads, "head_dim": case.head_dim,
            "layers": case.num_layers, "batch": case.batch}
    arrays = {}
    if prefill:
        nseq = min(case.batch, 8) if run.chunked else case.batch
        qs = case.query_start[:nseq + 1].astype(np.int64)
        arrays["q"] = q_all[qs[0]:qs[-1]]
        arrays["query_start"] = qs - qs[0]
        meta.update(kind="prefill", what=f"first {nseq} of {case.batch} sequences")
    elif grouped:
        offs, shared = wl.table_groups(case.block_tables, case.context_lens)
        nseq = int(offs[-1])
        arrays["q"] = q_all[:nseq]
        arrays["group_offsets"] = offs.astype(np.int64)
        arrays["shared_blocks"] = shared.astype(np.int64)
        meta.update(kind="grouped", what=f"all {len(shared)} groups ({nseq} sequences)")
    else:
        nseq = case.batch
        arrays["q"] = q_all[:nseq]
        meta.update(kind="decode", what=f"all {nseq} sequences")
    k_small, v_small, tables = _sample_pools(case.block_tables[:nseq], run.kp, run.vp, torch)
    arrays.update(k_pool=k_small, v_pool=v_small, tables=tables,
                  lens=case.context_lens[:nseq].astype(np.int64))
    meta["layer"] = "layer 0 of the step" if case.q.ndim == 4 else "one layer"
    return arrays, meta


def cpu_baseline(run, torch):
    """The oracle, as it stands, timed on the host's cores on a bounded
    sample of the workload (``cpu_sample``).  It runs in a child process
    that never touches the GPU: the sample goes through .npy files, and the
    child spreads the oracle's work units (sequences, groups, or row ranges
    of a prefill) over a pool of forked workers with one BLAS thread each;
    a serial pass over a few units gives the single-core rate."""
    import shutil
    import subprocess
    import tempfile

    import numpy as np
    arrays, meta = cpu_sample(run, torch)
    tmp = tempfile.mkdtemp(prefix="pkv_cpu_baseline_")
    try:
        for name, a in arrays.items():
            np.save(os.path.join(tmp, name + ".npy"), np.ascontiguousarray(a))
        with open(os.path.join(tmp, "meta.json"), "w") as f:
            json.dump(meta, f)
        del arrays
        env = dict(os.environ)
        for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
            env[var] = "1"
        res = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-worker", tmp],
                             env=env, stdout=subprocess.PIPE, timeout=600, check=True, text=True)
        return json.loads(res.stdout.strip().splitlines()[-1])
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


# -- the CPU-baseline child process (no GPU) ---------------------------------

_W = {}


def _unit_work(i):
    """Run work unit i of the sample through the oracle; returns its wall
    seconds."""
    import numpy as np
    from oracle import paged_decode_ref, paged_prefill_ref
    a, meta, (lo, hi, r0, r1) = _W["arrays"], _W["meta"], _W["units"][i]
    t0 = time.perf_counter()
    if meta["kind"] == "prefill":
        qs = a["query_start"]
        n = int(qs[lo + 1] - qs[lo])
        ctx = int(a["lens"][lo])
        # rows r0 .. r1-1 of sequence lo: the same positions as a query set
        # of r1 - r0 rows over the context up to row r1 - 1
        rows = np.arange(qs[lo] + r0, qs[lo] + r1)
        paged_prefill_ref(a["q"][rows], a["k_pool"], a["v_pool"], a["tables"][lo:lo + 1],
                          np.array([max(ctx - n + r1, 0)]), np.array([0, r1 - r0]),
                          meta["scale"])
    elif meta["kind"] == "grouped":
        # sequences lo .. hi-1 with the tables and lengths the grouping
        # contract gives them (grouped_tables_ref, applied once to the sample)
        paged_decode_ref(a["q"][lo:hi], a["k_pool"], a["v_pool"], _W["g_tables"][lo:hi],
                         _W["g_lens"][lo:hi], meta["scale"])
    else:
        paged_decode_ref(a["q"][lo:hi], a["k_pool"], a["v_pool"], a["tables"][lo:hi],
                         a["lens"][lo:hi], meta["scale"])
    return time.perf_counter() - t0


def cpu_worker_main(tmp):
    """Child process: load the sample, time the oracle serially on a few
    units (single core), then on all units over the worker pool; print one
    JSON object."""
    import multiprocessing as mp

    import numpy as np
    with open(os.path.join(tmp, "meta.json")) as f:
        meta = json.load(f)
    arrays = {n[:-4]: np.load(os.path.join(tmp, n), mmap_mode="r")
              for n in os.listdir(tmp) if n.endswith(".npy")}
    H, D = meta["heads"], meta["head_dim"]
    workers = cpu_workers()
    lens = np.asarray(arrays["lens"], dtype=np.int64)
    units, work = [], []               # (lo, hi, r0, r1), and its measure
    if meta["kind"] == "prefill":
        qs = np.asarray(arrays["query_start"])
        rows_total = int(qs[-1])
        per = max(1, -(-rows_total // (4 * workers)))   # rows per unit
        for b in range(len(lens)):
            n = int(qs[b + 1] - qs[b])
            for r0 in range(0, n, per):
                units.append((b, b + 1, r0, min(n, r0 + per)))
                work.append(min(n, r0 + per) - r0)
        unit, scale = "tokens/s", 1.0
    else:
        per = max(1, -(-len(lens) // (4 * workers)))
        for lo in range(0, len(lens), per):
            units.append((lo, min(len(lens), lo + per), 0, 0))
            work.append(int(lens[lo:lo + per].sum()))
        unit, scale = "GB/s", 2 * H * D * 2 / 1e9
    _W.update(arrays=arrays, meta=meta, units=units)
    t_groups = 0.0
    if meta["kind"] == "grouped":
        # the grouping contract once (host work, timed and added to both
        # figures); the decode of its tables is split into sequence units
        from oracle import grouped_tables_ref
        t0 = time.perf_counter()
        g_tables, g_lens = grouped_tables_ref(arrays["tables"], lens, arrays["group_offsets"],
                                              arrays["shared_blocks"], 16)
        t_groups = time.perf_counter() - t0
        _W.update(g_tables=g_tables, g_lens=g_lens)
    # single core: units in order until about 3 s have passed
    t_one, w_one, n_one = t_groups, 0, 0
    for i in range(len(units)):
        t_one += _unit_work(i)
        w_one += work[i]
        n_one += 1
        if t_one >= 3.0:
            break
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        pool.map(int, range(workers))               # workers up before the clock starts
        t0 = time.perf_counter()
        pool.map(_unit_work, range(len(units)), chunksize=1)
        wall = time.perf_counter() - t0 + t_groups
    total = sum(work)
    seqs = len(lens)
    rec = {"value": total * scale / wall, "unit": unit, "cores": workers, "kind": "oracle",
           "sample": f"{meta['what']} ({total} {'query rows' if unit == 'tokens/s' else 'context tokens'}"
                     f"), {meta['layer']}, float64 numpy oracle in {len(units)} work units over "
                     f"{workers} worker processes (1 BLAS thread each), {wall:.2f} s wall",
           "single_core": {"value": w_one * scale / t_one, "unit": unit,
                           "sample": f"first {n_one} of {len(units)} work units, one process, "
                                     f"{t_one:.2f} s"},
           "host_cpus_visible": len(os.sched_getaffinity(0))}
    if unit == "GB/s":
        rec["seq_layers_per_s"] = seqs / wall
    print(json.dumps(rec), flush=True)


def mark(torch, events):
    """Record a timing event on torch's current stream (the stream the calls
    are launched on) into ``events``; nothing when ``events`` is None."""
    if events is not None:
        ev = torch.cuda.Event(enable_timing=True)
        ev.record()
        events.append(ev)


class Run:
    """One benchmark workload: what a step does and how to count it."""

    def __init__(self, **kw):
        self.__dict__.update(kw)


def setup_batch(torch, dev, wl, args, batch, seed):
    """One layer; each step appends one token per sequence and decodes."""
    from paged_kv_cache_03_amd import (default_partition, kv_append, pa_decode, pa_decode_append,
                                       pa_decode_workspace_size)
    case = wl.gpt_batch(batch, seed=seed, append=True, fill=False)
    B, H, D = case.batch, case.num_heads, case.head_dim
    kp = wl.device_pool(torch, case, 0, 0, dev)
    vp = wl.device_pool(torch, case, 0, 1, dev)
    t = lambda a: torch.from_numpy(a).to(dev)
    q, tables, lens = t(case.q), t(case.block_tables), t(case.context_lens)
    k_new, v_new, slots = t(case.k_new), t(case.v_new), t(case.slot_mapping)
    out = torch.empty_like(q)
    max_ctx = case.max_context
    part = args.partition
    strategy = "partitioned" if (part or default_partition(B, H, D, max_ctx)) else "flat"
    ws = torch.empty(max(1, pa_decode_workspace_size(B, H, D, max_ctx, part)), dtype=torch.uint8,
                     device=dev)
    kv_bytes, algo_bytes = algorithmic_bytes(case.context_lens, H, D)
    fused = strategy == "flat" and not args.separate_append

    if fused:
        # the call also reads the new K/V rows and writes them to the pools
        algo_bytes += 2 * (2 * B * H * D * 2)

        def step(events):
            mark(torch, events)
            pa_decode_append(q, k_new, v_new, kp, vp, tables, lens, case.scale, out,
                             max_context_len=max_ctx, workspace=ws)
            mark(torch, events)
    else:
        def step(events):
            kv_append(k_new, v_new, slots, kp, vp)
            mark(torch, events)
            pa_decode(q, kp, vp, tables, lens, case.scale, out, max_context_len=max_ctx,
                      workspace=ws, partition_tokens=part)
            mark(torch, events)

    how = ("kv_append of 1 token/sequence fused into pa_decode (pa_decode_append) per step"
           if fused else "kv_append of 1 token/sequence + pa_decode per step")
    return Run(case=case, kp=kp, vp=vp, step=step, seqs_per_step=B, kv_bytes=kv_bytes,
               algo_bytes=algo_bytes, strategy=strategy, part=part, extra={}, fused=fused,
               timed_calls=1 if fused else 0, calls_per_call=1,
               call=None if fused else (lambda: pa_decode(q, kp, vp, tables, lens, case.scale, out,
                                                          max_context_len=max_ctx, workspace=ws,
                                                          partition_tokens=part)),
               config={"workload": f"one layer, batch {B}, 32 heads x 128 dims fp16, 16-token "
                                   "blocks, contexts prompt U[32,256] + geometric(mean 500) "
                                   f"capped at 2048, {how}",
                       "batch": B, "heads": H, "head_dim": D, "block_tokens": 16,
                       "context_tokens": case.kv_tokens(), "max_context": max_ctx,
                       "num_blocks": case.num_blocks, "strategy": strategy,
                       "partition_tokens": part, "seed": seed})


def grouped_decoder(torch, dev, wl, case, max_ctx):
    """pa_decode_grouped over the case's tables, grouped as they share blocks
    (consecutive sequences with a common first block, at most 16 a group)."""
    from paged_kv_cache_03_amd import pa_decode_grouped, pa_decode_grouped_workspace_size
    offs, shared = wl.table_groups(case.block_tables, case.context_lens)
    B, H, D = case.batch, case.num_heads, case.head_dim
    ws = torch.empty(pa_decode_grouped_workspace_size(B, H, D, max_ctx, len(shared)),
                     dtype=torch.uint8, device=dev)
    offs_t = torch.from_numpy(offs).to(dev)
    shared_t = torch.from_numpy(shared).to(dev)

    def decode(q, kp, vp, tables, lens, out):
        pa_decode_grouped(q, kp, vp, tables, lens, offs_t, shared_t, case.scale, out,
                          max_context_len=max_ctx, workspace=ws)

    info = {"groups": len(shared), "shared_blocks_per_group": sorted(set(shared.tolist()))}
    return decode, info


def setup_shared_prefix(torch, dev, wl, args):
    """One layer, 100 sequences sharing a 1024-token prefix; each step copies
    the prefix's last block per sequence (copy-on-write) and decodes."""
    from paged_kv_cache_03_amd import cow_copy_blocks, pa_decode, pa_decode_workspace_size
    case = wl.shared_prefix(fill=False)
    B, H, D = case.batch, case.num_heads, case.head_dim
    kp = wl.device_pool(torch, case, 0, 0, dev)
    vp = wl.device_pool(torch, case, 0, 1, dev)
    t = lambda a: torch.from_numpy(a).to(dev)
    q, tables, lens, pairs = t(case.q), t(case.block_tables), t(case.context_lens), t(case.cow_pairs)
    out = torch.empty_like(q)
    max_ctx = case.max_context
    kv_bytes, algo_bytes = algorithmic_bytes(case.context_lens, H, D)
    import numpy as np
    used = np.unique(case.block_tables[case.block_tables >= 0])
    unique_bytes = int(used.size) * H * 16 * D * 2 * 2
    extra = {"unique_kv_bytes": unique_bytes}
    if args.decode == "flat":
        ws = torch.empty(max(1, pa_decode_workspace_size(B, H, D, max_ctx, args.partition)),
                         dtype=torch.uint8, device=dev)

        def decode(q, kp, vp, tables, lens, out):
            pa_decode(q, kp, vp, tables, lens, case.scale, out, max_context_len=max_ctx,
                      workspace=ws, partition_tokens=args.partition, keep_cached=True)
        extra.update(decode="pa_decode", keep_cached=True)
        strategy = "flat" if not args.partition else "partitioned"
    else:
        decode, info = grouped_decoder(torch, dev, wl, case, max_ctx)
        extra.update(decode="pa_decode_grouped", **info)
        strategy = "grouped"

    def step(events):
        cow_copy_blocks(pairs, [kp], [vp])
        mark(torch, events)
        decode(q, kp, vp, tables, lens, out)
        mark(torch, events)

    return Run(case=case, kp=kp, vp=vp, step=step, seqs_per_step=B, kv_bytes=kv_bytes,
               algo_bytes=algo_bytes, strategy=strategy, part=args.partition, extra=extra,
               call=lambda: decode(q, kp, vp, tables, lens, out), calls_per_call=1,
               config={"workload": "one layer, batch 100, a 1024-token prefix in 64 shared "
                                   "blocks + private suffix U[0,500]; per step copy-on-write of "
                                   "the prefix's last block for each sequence + decode",
                       "batch": B, "heads": H, "head_dim": D, "block_tokens": 16,
                       "context_tokens": case.kv_tokens(), "max_context": max_ctx,
                       "num_blocks": case.num_blocks, "seed": 3})


def setup_full_step(torch, dev, wl, args, beams):
    """32 layers x 200 sequences x 2048 tokens; per step (beam groups:
    copy-on-write of each beam's last block in every layer, then) per layer
    append one token per sequence and decode."""
    from paged_kv_cache_03_amd import (cow_copy_blocks, kv_append, pa_decode, pa_decode_append,
                                       pa_decode_workspace_size)
    case = wl.full_step(beams=beams)
    B, H, D, L = case.batch, case.num_heads, case.head_dim, case.num_layers
    per_pool = case.num_blocks * H * 16 * D * 2
    free, _ = torch.cuda.mem_get_info(dev)
    distinct = max(1, min(L, int((free - (8 << 30)) // (2 * per_pool))))
    log(f"{L} layers, {distinct} distinct layer pools of {2 * per_pool / 2**30:.2f} GiB")
    pools = [(wl.device_pool(torch, case, l, 0, dev), wl.device_pool(torch, case, l, 1, dev))
             for l in range(distinct)]
    t = lambda a: torch.from_numpy(a).to(dev)
    qs = [t(case.q[l]) for l in range(L)]
    kn = [t(case.k_new[l]) for l in range(L)]
    vn = [t(case.v_new[l]) for l in range(L)]
    tables, lens, slots = t(case.block_tables), t(case.context_lens), t(case.slot_mapping)
    pairs = t(case.cow_pairs) if case.cow_pairs is not None else None
    out = torch.empty_like(qs[0])
    ws = torch.empty(max(1, pa_decode_workspace_size(B, H, D, 2048, args.partition)),
                     dtype=torch.uint8, device=dev)
    kv_layer, algo_layer = algorithmic_bytes(case.context_lens, H, D)
    layer_pools = [pools[l % distinct] for l in range(L)]
    grouped = beams > 1 and args.decode != "flat" or args.decode == "grouped"
    # the single-query decode takes each layer's append in the same call
    # (pa_decode_append), as the headline step does
    fused = not grouped and not args.partition and not args.separate_append
    if grouped:
        decode, info = grouped_decoder(torch, dev, wl, case, 2048)
        dec_extra = {"decode": "pa_decode_grouped", **info}
    elif fused:
        dec_extra = {"decode": "pa_decode_append", "keep_cached": beams > 1}
        algo_layer += 2 * (2 * B * H * D * 2)          # new rows read and written
    else:
        def decode(q, kp, vp, tables, lens, out):
            pa_decode(q, kp, vp, tables, lens, case.scale, out, max_context_len=2048,
                      workspace=ws, partition_tokens=args.partition, keep_cached=beams > 1)
        dec_extra = {"decode": "pa_decode", "keep_cached": beams > 1}

    def step(events):
        if pairs is not None:
            cow_copy_blocks(pairs, [p[0] for p in pools], [p[1] for p in pools])
        for l in range(L):
            kp, vp = layer_pools[l]
            if fused:
                mark(torch, events)
                pa_decode_append(qs[l], kn[l], vn[l], kp, vp, tables, lens, case.scale, out,
                                 max_context_len=2048, workspace=ws, keep_cached=beams > 1)
            else:
                kv_append(kn[l], vn[l], slots, kp, vp)
                mark(torch, events)
                decode(qs[l], kp, vp, tables, lens, out)
            mark(torch, events)

    def call():                        # every layer's decode alone, back to back
        for l in range(L):
            kp, vp = layer_pools[l]
            decode(qs[l], kp, vp, tables, lens, out)

    import numpy as np
    used = np.unique(case.block_tables)
    return Run(case=case, kp=pools[0][0], vp=pools[0][1], step=step, seqs_per_step=B * L,
               call=None if fused else call, calls_per_call=L,
               kv_bytes=kv_layer * L, algo_bytes=algo_layer, fused=fused,
               timed_calls=L if fused and pairs is None else 0,
               strategy="grouped" if grouped else "flat" if not args.partition else "partitioned",
               part=args.partition,
               extra={"layers": L, "distinct_layer_pools": distinct, **dec_extra,
                      "unique_kv_bytes": int(used.size) * H * 16 * D * 2 * 2},
               config={"workload": f"full decode step: {L} layers x batch {B} x 2048 tokens, "
                                   "32 heads x 128 dims fp16; per layer "
                                   + ("append fused into the decode (pa_decode_append)"
                                      if fused else "kv_append + decode")
                                   + (f"; {beams}-beam groups sharing all but the last block, "
                                      "copy-on-write of the last block per beam" if beams > 1
                                      else ""),
                       "batch": B, "layers": L, "heads": H, "head_dim": D, "block_tokens": 16,
                       "context_tokens_per_layer": case.kv_tokens(), "num_blocks": case.num_blocks,
                       "beams": beams, "seed": 4})


MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix peak


def setup_vattention(torch, dev, wl, args):
    """The headline batch (200 sequences, one layer) on a contiguous KV cache
    in virtual memory with physical chunks mapped on demand (the vAttention
    alternative): per step one new token per sequence is written into its
    row and the contiguous decode runs.  The paged step on the same data is
    timed alongside, and the physical memory of both layouts is reported."""
    import time as _time

    import numpy as np
    from paged_kv_cache_03_amd import (VirtualKV, contig_decode, contig_decode_workspace_size,
                                       pa_decode)
    case = wl.gpt_batch(200, seed=2, append=True, fill=False)
    B, H, D, L = case.batch, case.num_heads, case.head_dim, 2048
    row = H * D * 2
    kp = wl.device_pool(torch, case, 0, 0, dev)
    vp = wl.device_pool(torch, case, 0, 1, dev)
    t = lambda a: torch.from_numpy(a).to(dev)
    q, lens, tables = t(case.q), t(case.context_lens), t(case.block_tables)
    vkv = VirtualKV(B, L, 1, H, D, chunk_bytes=args.vkv_chunk)
    t0 = _time.perf_counter()
    for b, n in enumerate(case.context_lens):
        vkv.grow(b, int(n))
    grow_s = _time.perf_counter() - t0
    # cached tokens (all but the last) copied from the paged pools
    NB = case.num_blocks
    tok = lambda pool: pool.view(NB, H, D // 8, 16, 8).permute(0, 3, 1, 2, 4).reshape(NB, 16, H, D)
    seq = np.concatenate([np.full(int(n) - 1, b, dtype=np.int32) for b, n in enumerate(case.context_lens)])
    pos = np.concatenate([np.arange(int(n) - 1, dtype=np.int32) for n in case.context_lens])
    blk = torch.from_numpy(case.block_tables[seq, pos // 16].astype(np.int64)).to(dev)
    slot = torch.from_numpy((pos % 16).astype(np.int64)).to(dev)
    vkv.append(0, tok(kp)[blk, slot].contiguous(), tok(vp)[blk, slot].contiguous(), t(seq), t(pos))
    torch.cuda.synchronize()
    new_seq = t(np.arange(B, dtype=np.int32))
    new_pos = t((case.context_lens - 1).astype(np.int32))
    kn, vn = t(case.k_new), t(case.v_new)
    out = torch.empty_like(q)
    ws = torch.empty(contig_decode_workspace_size(B, H, D, case.max_context), dtype=torch.uint8,
                     device=dev)

    def step(events):
        vkv.append(0, kn, vn, new_seq, new_pos)
        mark(torch, events)
        contig_decode(q, vkv, 0, lens, case.scale, out, max_context_len=case.max_context,
                      workspace=ws)
        mark(torch, events)

    # the paged decode on the same tokens, for comparison
    ref_out = torch.empty_like(q)
    for _ in range(5):
        pa_decode(q, kp, vp, tables, lens, case.scale, ref_out, max_context_len=case.max_context)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(50):
        pa_decode(q, kp, vp, tables, lens, case.scale, ref_out, max_context_len=case.max_context)
    e.record()
    torch.cuda.synchronize()
    paged_us = s.elapsed_time(e) / 50 * 1e3

    # the same rows in one ordinary allocation: the layout without the mapping
    from paged_kv_cache_03_amd import contig_decode_rows
    rows = torch.from_numpy(seq.astype(np.int64) * L + pos).to(dev)
    k_rows = torch.zeros((B * L, H, D), dtype=torch.float16, device=dev)
    v_rows = torch.zeros_like(k_rows)
    k_rows.index_copy_(0, rows, tok(kp)[blk, slot])
    v_rows.index_copy_(0, rows, tok(vp)[blk, slot])
    last = torch.from_numpy(np.arange(B, dtype=np.int64) * L + case.context_lens - 1).to(dev)
    k_rows.index_copy_(0, last, kn)
    v_rows.index_copy_(0, last, vn)
    for _ in range(5):
        contig_decode_rows(q, k_rows, v_rows, L, lens, case.scale, ref_out,
                           max_context_len=case.max_context, workspace=ws)
    torch.cuda.synchronize()
    s.record()
    for _ in range(50):
        contig_decode_rows(q, k_rows, v_rows, L, lens, case.scale, ref_out,
                           max_context_len=case.max_context, workspace=ws)
    e.record()
    torch.cuda.synchronize()
    plain_us = s.elapsed_time(e) / 50 * 1e3
    del k_rows, v_rows

    st = vkv.stats()
    ctx = case.context_lens.astype(np.int64)
    r16 = (ctx + 15) // 16 * 16
    mapped_at = lambda c: int(((r16 * row + c - 1) // c * c).sum()) * 2
    paged_bytes = int(((ctx + 15) // 16).sum()) * 16 * row * 2
    kv_bytes, algo_bytes = algorithmic_bytes(case.context_lens, H, D)
    written = int(ctx.sum()) * row * 2
    extra = {
        "decode": "pkv_contig_decode (contiguous rows in virtual memory)",
        "paged_decode_us_same_tokens": round(paged_us, 3),
        "contig_decode_us_ordinary_allocation": round(plain_us, 3),
        "memory": {
            "written_kv_bytes": written,
            "paged_16_token_blocks_bytes": paged_bytes,
            "virtual_mapped_bytes": int(st["mapped_bytes"]),
            "virtual_chunk_bytes": int(st["chunk_bytes"]),
            "virtual_mapped_bytes_by_chunk": {str(c): mapped_at(c)
                                              for c in (64 << 10, 256 << 10, 2 << 20)},
            "naive_max_context_bytes": B * L * row * 2,
            "reserved_virtual_bytes": int(st["reserved_bytes"]),
        },
        "mapping": {"granularity": int(st["granularity"]), "map_calls": int(st["map_calls"]),
                    "us_per_map_call": round(1e6 * st["map_seconds"] / max(st["map_calls"], 1), 1),
                    "grow_all_s": round(grow_s, 4)},
    }
    return Run(case=case, kp=kp, vp=vp, step=step, seqs_per_step=B, kv_bytes=kv_bytes,
               algo_bytes=algo_bytes, strategy="contiguous", part=0, extra=extra, vkv=vkv,
               config={"workload": "one layer, batch 200, 32 heads x 128 dims fp16, contexts "
                                   "prompt U[32,256] + geometric(mean 500) capped at 2048, in a "
                                   "contiguous virtual-memory cache mapped in "
                                   f"{args.vkv_chunk} B chunks; per step append of 1 "
                                   "token/sequence + contiguous decode",
                       "batch": B, "heads": H, "head_dim": D, "max_context": L,
                       "context_tokens": case.kv_tokens(), "seed": 2})


def setup_prefill(torch, dev, wl, args, chunked):
    """One layer of prefill: per step the new tokens' keys and values are
    written to their slots and every new token attends causally over its
    sequence.  Prompts: 200 sequences of U[32, 256] tokens, one
    pa_prefill_append call (--separate-append: kv_append, then pa_prefill);
    chunked: 32 sequences, a 512-token chunk over 1536 cached tokens,
    kv_append then pa_prefill, the faster of the two there (--fused-append:
    one pa_prefill_append call)."""
    from paged_kv_cache_03_amd import kv_append, pa_prefill, pa_prefill_append
    import numpy as np
    case = wl.prefill(32, seed=7, cached=1536, chunk=512, fill=False) if chunked else \
        wl.prefill(fill=False)
    H, D = case.num_heads, case.head_dim
    kp = wl.device_pool(torch, case, 0, 0, dev)
    vp = wl.device_pool(torch, case, 0, 1, dev)
    t = lambda a: torch.from_numpy(a).to(dev)
    q, tables, lens, qs = t(case.q), t(case.block_tables), t(case.context_lens), t(case.query_start)
    kn, vn, slots = t(case.k_new), t(case.v_new), t(case.slot_mapping)
    out = torch.empty_like(q)
    max_ctx = case.max_context

    fused = args.fused_append if chunked else not args.separate_append

    def step(events):
        if not fused:
            kv_append(kn, vn, slots, kp, vp)
        mark(torch, events)
        if fused:
            pa_prefill_append(q, kn, vn, kp, vp, tables, lens, qs, case.scale, out,
                              max_context_len=max_ctx)
        else:
            pa_prefill(q, kp, vp, tables, lens, qs, case.scale, out, max_context_len=max_ctx)
        mark(torch, events)

    n = np.diff(case.query_start).astype(np.int64)
    ctx = case.context_lens.astype(np.int64)
    # causal (query, key) pairs: a chunk of n over c cached tokens sees c*n + n(n+1)/2
    pairs = int(((ctx - n) * n + n * (n + 1) // 2).sum())
    flops = 4 * H * D * pairs                          # q.k and p.v, 2 flops per multiply-add
    kv_bytes = int(ctx.sum()) * H * D * 2 * 2          # every cached token's K and V once
    io_bytes = int(n.sum()) * H * D * 2 * 2            # q read, out written
    # fused: the new tokens' K and V are read from their rows instead of the
    # pools (the same count) and written to the pools once
    write_bytes = int(np.maximum(np.minimum(n, ctx), 0).sum()) * H * D * 2 * 2 if fused else 0
    rows = int(n.sum())
    return Run(case=case, kp=kp, vp=vp, step=step, seqs_per_step=case.batch, kv_bytes=kv_bytes,
               algo_bytes=kv_bytes + io_bytes + write_bytes, strategy="prefill", part=0,
               chunked=chunked, timed_calls=1 if fused else 0,
               call=None if fused else (lambda: pa_prefill(q, kp, vp, tables, lens, qs, case.scale,
                                                           out, max_context_len=max_ctx)),
               calls_per_call=1,
               prefill={"rows": rows, "flops": flops, "pairs": pairs,
                        "kernel": "pa_prefill_append" if fused else "pa_prefill"},
               extra={"query_rows": rows, "causal_pairs": pairs},
               config={"workload": ("one layer, 32 sequences x (1536 cached + 512-token chunk)"
                                    if chunked else "one layer, 200 prompts of U[32,256] tokens")
                                   + ", 32 heads x 128 dims fp16; per step "
                                   + ("pa_prefill_append (the new tokens written to their pages "
                                      "and attended causally in one call)" if fused else
                                      "kv_append of the new tokens + causal pa_prefill"),
                       "batch": case.batch, "heads": H, "head_dim": D, "block_tokens": 16,
                       "query_rows": rows, "context_tokens": case.kv_tokens(),
                       "max_context": max_ctx, "num_blocks": case.num_blocks,
                       "seed": case.meta["seed"]})


def measure(torch, dev, wl, args, name, steps, warmup, cold_reps=0, probe=False, cpu=True):
    """Set up workload ``name``, run ``warmup`` untimed steps and ``steps``
    timed ones, and return its bench record (without printing it)."""
    import numpy as np

    if name == "batch200":
        run = setup_batch(torch, dev, wl, args, 200, 2)
    elif name == "batch10":
        run = setup_batch(torch, dev, wl, args, 10, 1)
    elif name == "shared_prefix":
        run = setup_shared_prefix(torch, dev, wl, args)
    elif name == "vattention":
        run = setup_vattention(torch, dev, wl, args)
    elif name.startswith("prefill"):
        run = setup_prefill(torch, dev, wl, args, name == "prefill_chunked")
    else:
        run = setup_full_step(torch, dev, wl, args, 4 if name == "beam_step" else 1)
    log(f"workload {name}: {run.config}")

    for _ in range(warmup):
        run.step(None)
    torch.cuda.synchronize()
    log(f"warmup {warmup} done")

    # A step made only of the timed call(s) is timed with one pair of events
    # around all the steps: an event recorded between calls costs about 7 us
    # of GPU time per step here.  Other steps record an event pair around
    # each timed call.
    only = getattr(run, "timed_calls", 0)
    events = None if only else []
    first, last = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    first.record()
    for i in range(steps):
        run.step(events)
    last.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"timed {steps} steps in {elapsed * 1e3:.2f} ms")
    if only:
        dec_ms = [first.elapsed_time(last) / (steps * only)] * (steps * only)
    else:
        dec_ms = [events[i].elapsed_time(events[i + 1]) for i in range(0, len(events), 2)]
    dec_avg_s = float(np.mean(dec_ms)) / 1e3
    ms_per_step = elapsed * 1e3 / steps

    step_gbs = run.kv_bytes / (ms_per_step / 1e3) / 1e9
    kv_per_call = run.kv_bytes / (len(dec_ms) / steps)
    dec_gbs = kv_per_call / dec_avg_s / 1e9
    achieved = run.algo_bytes / dec_avg_s / 1e9
    headline = name == "batch200" and getattr(run, "fused", False)
    result = {
        "metric": "pa_decode K/V GB/s (% MI355X HBM peak) + seq-layers/s at batch 200",
        "value": round(step_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": run.config,
        "pct_hbm_peak": round(100 * step_gbs / HBM_PEAK_GBS, 2),
        "seq_layers_per_s": round(run.seqs_per_step / (ms_per_step / 1e3), 1),
        "pa_decode_us": round(dec_avg_s * 1e6, 3),
        "pa_decode_us_median": round(float(np.median(dec_ms)) * 1e3, 3),
        "pa_decode_us_p90": round(float(np.percentile(dec_ms, 90)) * 1e3, 3),
        "call_timing": ("one event pair around the timed steps (calls back to back)" if only
                        else "an event pair around each call"),
        "pa_decode_kv_gbs": round(dec_gbs, 2),
        "pa_decode_pct_hbm_peak": round(100 * dec_gbs / HBM_PEAK_GBS, 2),
        "roofline": {
            "kernel": ("pa_decode_append (fused append + decode kernel, merge kernel; one call)"
                       if getattr(run, "fused", False) else
                       "pa_decode_grouped (grouped decode + merge kernels, one call)"
                       if run.extra.get("decode") == "pa_decode_grouped" else
                       "pa_decode (decode + merge kernels, one call)"),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "bytes_per_launch": run.algo_bytes,
            "traffic": measured_traffic() if headline else None,
        },
    }
    if only:      # one average over all calls: no per-call spread
        del result["pa_decode_us_median"], result["pa_decode_us_p90"]
    elif getattr(run, "call", None) is not None:
        # The timed call alone, repeated back to back between one event pair
        # (the step's other kernels and the per-call events left out): the
        # call's own rate, next to the in-step figure the roofline uses.
        for _ in range(3):
            run.call()
        reps = max(steps, 5)
        first.record()
        for _ in range(reps):
            run.call()
        last.record()
        torch.cuda.synchronize()
        b2b_s = first.elapsed_time(last) / 1e3 / (reps * run.calls_per_call)
        result["pa_decode_us_back_to_back"] = round(b2b_s * 1e6, 3)
    result.update(run.extra)
    pf = getattr(run, "prefill", None)
    if pf is not None:
        # prefill: the bound is whichever of HBM bytes and matrix flops takes longer
        tflops = pf["flops"] / dec_avg_s / 1e12
        t_hbm = run.algo_bytes / (HBM_PEAK_GBS * 1e9)
        t_mfma = pf["flops"] / (MFMA_F16_PEAK_TFLOPS * 1e12)
        result["metric"] = "pa_prefill tokens/s, TFLOP/s and GB/s (one layer)"
        result["value"] = round(pf["rows"] / (ms_per_step / 1e3), 1)
        result["unit"] = "tokens/s"
        result["pa_prefill_us"] = result.pop("pa_decode_us")
        if not only:
            result["pa_prefill_us_median"] = result.pop("pa_decode_us_median")
            result["pa_prefill_us_p90"] = result.pop("pa_decode_us_p90")
        if "pa_decode_us_back_to_back" in result:
            result["pa_prefill_us_back_to_back"] = result.pop("pa_decode_us_back_to_back")
        result["pa_prefill_tflops"] = round(tflops, 2)
        result["pa_prefill_gbs"] = round(achieved, 2)
        for k in ("pa_decode_kv_gbs", "pa_decode_pct_hbm_peak", "pct_hbm_peak"):
            result.pop(k, None)
        if t_mfma >= t_hbm:
            result["roofline"].update(kernel=pf["kernel"], bound="mfma", unit="TFLOP/s",
                                      achieved=round(tflops, 2), peak=MFMA_F16_PEAK_TFLOPS,
                                      frac=round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                                      flops_per_launch=pf["flops"])
        else:
            result["roofline"].update(kernel=pf["kernel"])
    if run.extra.get("unique_kv_bytes", kv_per_call) < kv_per_call:   # each distinct block once
        result["pa_decode_unique_kv_gbs"] = round(run.extra["unique_kv_bytes"] / dec_avg_s / 1e9, 2)
        # blocks shared by several sequences: HBM sees each once, so the
        # roofline counts the distinct blocks (the logical rate stays above)
        unique_call = run.algo_bytes - kv_per_call + run.extra["unique_kv_bytes"]
        result["roofline"].update(
            kernel=result["roofline"]["kernel"] + ", distinct blocks",
            achieved=round(unique_call / dec_avg_s / 1e9, 2),
            frac=round(unique_call / dec_avg_s / 1e9 / HBM_PEAK_GBS, 4),
            bytes_per_launch=int(unique_call), logical_bytes_per_launch=run.algo_bytes)
    b2b_us = result.get("pa_decode_us_back_to_back", result.get("pa_prefill_us_back_to_back"))
    if b2b_us:                         # the same roofline on the back-to-back call time
        rf = result["roofline"]
        a = (pf["flops"] / (b2b_us * 1e-6) / 1e12 if rf["unit"] == "TFLOP/s"
             else rf["bytes_per_launch"] / (b2b_us * 1e-6) / 1e9)
        rf["achieved_back_to_back"] = round(a, 2)
        rf["frac_back_to_back"] = round(a / rf["peak"], 4)

    if cold_reps > 0 and name in ("batch200", "batch10", "shared_prefix",
                                                "vattention", "prefill_prompt",
                                                "prefill_chunked"):
        # The timed steps above run warm: a working set under 256 MB (batch 10)
        # or shared blocks (the prefix) can be served by the MALL between
        # steps.  Here every call starts after 1 GiB of unrelated writes.
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cold = []
        for i in range(cold_reps):
            scratch.fill_(i & 0xFF)
            ev = []
            run.step(ev)
            torch.cuda.synchronize()
            cold.append(ev[0].elapsed_time(ev[1]))
        del scratch
        key = "pa_prefill" if pf is not None else "pa_decode"
        result[key + "_us_cold_median"] = round(float(np.median(cold)) * 1e3, 3)
        result[key + "_us_cold_p90"] = round(float(np.percentile(cold, 90)) * 1e3, 3)
        result[key + "_cold_reps"] = cold_reps

    if probe:
        hp = hbm_probe(torch, dev)
        result["hbm_probe"] = hp
        result["roofline"]["achievable_gather_gbs"] = hp["gather_4k_gbs"]
        result["roofline"]["frac_of_achievable"] = round(achieved / hp["gather_4k_gbs"], 4)

    if (name == "prefill_prompt" and pf is not None and pf["kernel"] == "pa_prefill_append"
            and not args.no_hbm_probe):
        # reads and writes in equal parts: the reference is a plain copy's rate
        cp = copy_probe(torch, dev)
        result["roofline"]["achievable_copy_gbs"] = cp
        result["roofline"]["frac_of_achievable"] = round(result["roofline"]["achieved"] / cp, 4)

    if args.copy_probe:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(10):
            dst.copy_(src)
        e.record()
        torch.cuda.synchronize()
        t = s.elapsed_time(e) / 10 / 1e3
        result["copy_probe"] = {"bytes_read": n, "bytes_written": n,
                                "gbs_read_plus_write": round(2 * n / t / 1e9, 1)}
        del src, dst

    if cpu:
        log(f"{name}: timing the oracle on a sample of the workload (cpu baseline)")
        result["cpu_baseline"] = cpu_baseline(run, torch)
        log(f"cpu baseline: {result['cpu_baseline']['sample']}")
    del run
    return result


def main():
    args = parse()
    if args.cpu_worker:
        cpu_worker_main(args.cpu_worker)
        return
    if args.traffic_from:
        write_traffic_record(*args.traffic_from)
        return
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; the library runs on one GPU "
              "(there is no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    import torch

    import workloads as wl
    from paged_kv_cache_03_amd import load_library

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    load_library()   # fails loudly when the HIP library is not built
    dev = torch.device("cuda:0")
    log(f"device {torch.cuda.get_device_name(0)} "
        f"({torch.cuda.get_device_properties(0).gcnArchName})")
    if args.lds_probe:
        print(json.dumps({"lds_read_probe": lds_probe(torch, dev)}), flush=True)
        return

    headline = args.workload == "batch200"
    result = measure(torch, dev, wl, args, args.workload, args.steps, args.warmup,
                     cold_reps=args.cold_reps, probe=headline and not args.no_hbm_probe,
                     cpu=not args.no_cpu_baseline)
    if headline and not args.no_extras:
        # the other workloads, each timed in the same run and summarised
        # inside the one line
        result["other_workloads"] = {}
        for name, steps, warmup in EXTRA_WORKLOADS:
            torch.cuda.empty_cache()
            rec = measure(torch, dev, wl, default_args(), name, steps, warmup,
                          cold_reps=args.cold_reps if name in ONE_LAYER else 0,
                          cpu=not args.no_cpu_baseline)
            result["other_workloads"][name] = summarise(rec)
            log(f"{name}: {json.dumps(result['other_workloads'][name]['roofline'])}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
