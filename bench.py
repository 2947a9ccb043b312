"""Throughput of the paged-decode hot path on one MI355X.

One step = one pass of the hot path over one batch: append one new token per
sequence into its slot (kv_append), then decode every sequence over its
whole context (pa_decode: partition kernel + merge kernel).  The workload is
one layer of a GPT-style model, batch 200, 32 heads x 128 dims, fp16,
16-token blocks, contexts = prompt U[32,256] + response geometric(mean 500)
capped at 2048, pool = blocks needed + 10% free, tables from a shuffled free
list (seed 2).  Inputs are resident in HBM before the timed region.

Prints one JSON line.  ``--gpus`` above 1 is refused: this build runs on one
GPU.
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
KV_BYTES_PER_TOKEN_LAYER = None  # set from the shape: 2 * H * D * 2


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--partition", type=int, default=0, help="partition tokens (0 = default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=0,
                    help="sequences in the oracle sample (0 = sized to ~15 s)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain device copy of known size (counter calibration)")
    return ap.parse_args()


def algorithmic_bytes(lens, H, D):
    """Per decode launch: K and V of every context token, q in and out, the
    block-table entries read, the context length."""
    lens = [int(x) for x in lens]
    kv = sum(lens) * 2 * H * D * 2
    qo = len(lens) * H * D * 2 * 2
    tab = sum(4 * math.ceil(n / 16) + 4 for n in lens)
    return kv, kv + qo + tab


def cpu_baseline(case, kp, vp, torch, budget_s=15.0, nseq=0):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np
    from oracle import paged_decode_ref
    order = list(range(case.batch))
    # pick a sample whose tokens are proportional to the budget; start small
    sample = order[: (nseq or 16)]
    ids = np.unique(case.block_tables[sample].reshape(-1))
    ids = ids[ids >= 0]
    remap = np.full(case.num_blocks, -1, dtype=np.int32)
    remap[ids] = np.arange(len(ids), dtype=np.int32)
    idx = torch.from_numpy(ids.astype(np.int64)).to(kp.device)
    k_small = kp.index_select(0, idx).cpu().numpy()
    v_small = vp.index_select(0, idx).cpu().numpy()
    tables = np.where(case.block_tables[sample] >= 0,
                      remap[np.maximum(case.block_tables[sample], 0)], -1).astype(np.int32)
    lens = case.context_lens[sample]
    w0, c0 = time.perf_counter(), time.process_time()
    paged_decode_ref(case.q[sample], k_small, v_small, tables, lens, case.scale)
    wall, cpu = time.perf_counter() - w0, time.process_time() - c0
    if not nseq and wall < budget_s / 4 and len(sample) < case.batch:
        # scale the sample up to roughly the budget, within the batch
        more = min(case.batch, int(len(sample) * budget_s / max(wall, 1e-3)))
        return cpu_baseline(case, kp, vp, torch, budget_s, nseq=max(more, len(sample) + 1))
    tokens = int(lens.astype(np.int64).sum())
    kv_bytes = tokens * 2 * case.num_heads * case.head_dim * 2
    return {
        "value": kv_bytes / wall / 1e9,
        "unit": "GB/s",
        "seq_layers_per_s": len(sample) / wall,
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"first {len(sample)} of {case.batch} sequences ({tokens} context tokens), "
                  f"one layer, float64 numpy oracle, {wall:.1f} s wall",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; this build measures one GPU "
              "(every GPU box here has one).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_03_amd import (kv_append, load_library, pa_decode,
                                       pa_decode_workspace_size, default_partition)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    load_library()   # fails loudly when the HIP library is not built
    dev = torch.device("cuda:0")
    log(f"device {torch.cuda.get_device_name(0)} "
        f"({torch.cuda.get_device_properties(0).gcnArchName})")

    case = wl.gpt_batch(200, seed=2, append=True, fill=False)
    B, H, D = case.batch, case.num_heads, case.head_dim
    kp = wl.device_pool(torch, case, 0, 0, dev)
    vp = wl.device_pool(torch, case, 0, 1, dev)
    q = torch.from_numpy(case.q).to(dev)
    tables = torch.from_numpy(case.block_tables).to(dev)
    lens = torch.from_numpy(case.context_lens).to(dev)
    k_new = torch.from_numpy(case.k_new).to(dev)
    v_new = torch.from_numpy(case.v_new).to(dev)
    slots = torch.from_numpy(case.slot_mapping).to(dev)
    out = torch.empty_like(q)
    max_ctx = case.max_context
    part = args.partition            # 0: the library's default plan
    strategy = "partitioned" if (part or default_partition(B, H, D, max_ctx)) else "flat"
    ws = torch.empty(max(1, pa_decode_workspace_size(B, H, D, max_ctx, part)), dtype=torch.uint8,
                     device=dev)
    kv_bytes, algo_bytes = algorithmic_bytes(case.context_lens, H, D)
    log(f"workload: B={B} H={H} D={D} blocks={case.num_blocks} tokens={case.kv_tokens()} "
        f"max_ctx={max_ctx} strategy={strategy} partition={part} kv_bytes={kv_bytes}")

    def step(ev=None):
        kv_append(k_new, v_new, slots, kp, vp)
        if ev is not None:
            ev[0].record()
        pa_decode(q, kp, vp, tables, lens, case.scale, out, max_context_len=max_ctx,
                  workspace=ws, partition_tokens=part)
        if ev is not None:
            ev[1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {elapsed * 1e3:.2f} ms")
    dec_ms = [s.elapsed_time(e) for s, e in events]
    dec_avg_s = float(np.mean(dec_ms)) / 1e3
    ms_per_step = elapsed * 1e3 / args.steps

    step_gbs = kv_bytes / (ms_per_step / 1e3) / 1e9
    dec_gbs = kv_bytes / dec_avg_s / 1e9
    achieved = algo_bytes / dec_avg_s / 1e9
    result = {
        "metric": "pa_decode K/V GB/s (% MI355X HBM peak) + seq-layers/s at batch 200",
        "value": round(step_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "one layer, batch 200, 32 heads x 128 dims fp16, 16-token blocks, "
                        "contexts prompt U[32,256] + geometric(mean 500) capped at 2048, "
                        "kv_append of 1 token/sequence + pa_decode per step",
            "batch": B, "heads": H, "head_dim": D, "block_tokens": 16,
            "context_tokens": case.kv_tokens(), "max_context": max_ctx,
            "num_blocks": case.num_blocks, "strategy": strategy, "partition_tokens": part,
            "seed": 2,
        },
        "pct_hbm_peak": round(100 * step_gbs / HBM_PEAK_GBS, 2),
        "seq_layers_per_s": round(B / (ms_per_step / 1e3), 1),
        "pa_decode_us": round(dec_avg_s * 1e6, 3),
        "pa_decode_kv_gbs": round(dec_gbs, 2),
        "pa_decode_pct_hbm_peak": round(100 * dec_gbs / HBM_PEAK_GBS, 2),
        "roofline": {
            "kernel": "pa_decode (decode + merge kernels, one call)",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "bytes_per_launch": algo_bytes,
            "traffic": None,
        },
    }

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

    if not args.no_cpu_baseline:
        log("timing the oracle on a sample of the workload (cpu baseline)")
        result["cpu_baseline"] = cpu_baseline(case, kp, vp, torch, nseq=args.cpu_seqs)
        log(f"cpu baseline: {result['cpu_baseline']['sample']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
