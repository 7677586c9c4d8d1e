#!/usr/bin/env python3
"""Benchmark: paged GQA decode attention, KV-read HBM bandwidth on one MI355X.

One step = one call of attn_decode_fwd (plan + split kernel [+ combine]) over
the paged bf16 decode workload: batch 32, Hq 32 / Hkv 8, head_dim 128,
q_len 1, 16-key pages, cache_seqlens ~ U{900..1100}, shuffled block_table.
Inputs are resident in HBM before timing.  The KV cache is replicated into
several pools and the steps rotate over them, so each step reads KV that is
not in the 256 MiB last-level cache from the previous step.

value = algorithmic KV bytes per step (valid keys x Hkv x d x 2 x 2 B)
        / wall time per step, in GB/s.

Prints one JSON line (see --help for options).
"""
import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
METRIC = "KV-read HBM GB/s (% of MI355X peak) for paged GQA decode attention"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c3",
                    choices=["c3", "c4", "c5"],
                    help="c3: paged bf16 B32 Hq32/Hkv8 d128 L~1000 (default); "
                         "c4: B4 Hq32/Hkv4 L16384; c5: ragged fp16 B128 d64")
    ap.add_argument("--num-splits", type=int, default=0, help="0 = planner")
    ap.add_argument("--pools", type=int, default=4, help="KV pool copies rotated over")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, copy this many MiB device to device once (the "
                         "known-size copy that scales the HBM byte counters)")
    return ap.parse_args()


def make_workload(name):
    from split_kv_paged_amd import workloads as W
    return {"c3": W.c3_paged_gqa4, "c4": W.c4_long, "c5": W.c5_ragged}[name]()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from split_kv_paged_amd import api

    wl = make_workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[wl.dtype]

    def dev16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).to(dev)

    q = dev16(wl.q)
    pools = [(dev16(wl.k_cache), dev16(wl.v_cache)) for _ in range(max(1, args.pools))]
    bt = torch.from_numpy(wl.block_table).to(dev)
    sl = torch.from_numpy(wl.cache_seqlens).to(dev)
    max_L = wl.max_seqlen_k
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    plan = api.decode_plan(wl.batch, wl.q_len, wl.num_heads_q, wl.num_heads_kv, wl.head_dim,
                           wl.page_size, wl.block_table.shape[1], max_L, tdt,
                           num_splits=args.num_splits, num_cus=cus)
    out = torch.empty_like(q)
    lse = torch.empty((wl.batch, wl.num_heads_q, wl.q_len), dtype=torch.float32, device=dev)
    ws = (torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device=dev)
          if plan.workspace_bytes else None)
    stream = torch.cuda.current_stream(dev)

    # one prepared call per KV pool: the per-step host work is a single call
    # into the C ABI (which still plans and validates every time)
    calls = [api.PreparedDecode(q, kc, vc, bt, sl, num_splits=args.num_splits,
                                softmax_scale=wl.scale, max_seqlen_k=max_L, out=out, lse=lse,
                                workspace=ws, stream=stream) for kc, vc in pools]

    def step(i):
        calls[i % len(calls)]()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Two HIP events on the launch stream bracket the K launches; the host
    # enqueues faster than the GPU drains, so the launches run back to back
    # and (end - start) / K is the average launch duration.
    K = args.steps
    ev_start = torch.cuda.Event(enable_timing=True)
    ev_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_start.record(stream)
    for i in range(K):
        step(i)
    ev_end.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = (t1 - t0) / K
    launch_ms = ev_start.elapsed_time(ev_end) / K
    last = api.last_plan()

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    kv_bytes = wl.kv_bytes
    value = kv_bytes / wall / 1e9
    kern_s = launch_ms / 1e3
    achieved = kv_bytes / kern_s / 1e9
    qheads = wl.batch * wl.num_heads_q * wl.q_len

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds)

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) bf16 K/V/Q, shuffled page table)",
        "config": {
            "workload": wl.name, "batch": wl.batch, "q_len": wl.q_len,
            "num_heads_q": wl.num_heads_q, "num_heads_kv": wl.num_heads_kv,
            "head_dim": wl.head_dim, "page_size": wl.page_size,
            "kv_tokens": int(wl.cache_seqlens.sum()), "kv_bytes": kv_bytes,
            "num_splits": last.num_splits, "pack_gqa": last.pack_gqa,
            "grid": last.grid, "kv_pools": len(pools), "accumulate": "f32",
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "query_heads_per_s": round(qheads / wall, 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(wl.name, last.num_splits),
            "kernel_avg_us": round(kern_s * 1e6, 3),
            "kernels_per_launch": 1 + last.combine,
        },
    }
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec), flush=True)


def measured_traffic(workload, num_splits):
    """HBM bytes per launch from the committed counter summary of this
    workload, or None when there is none or the kernel sources changed since
    the counters were taken."""
    from split_kv_paged_amd import profiling
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        "hbm_traffic_%s.md" % workload)
    if not os.path.exists(path):
        return None
    v = profiling.read_traffic(path)
    if (v.get("workload") != workload or v.get("num_splits") != str(num_splits)
            or v.get("source_digest") != profiling.source_digest()):
        return None
    return int(float(v["traffic_bytes_per_launch"]))


def cpu_baseline(wl, budget_s):
    """The float64 oracle on the host cores, same workload, a bounded number
    of repetitions (about budget_s seconds)."""
    import numpy as np

    import oracle
    threads = oracle.default_threads()
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.cache_seqlens,
                               wl.dtype, scale=wl.scale, nthreads=threads)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 20:
            break
    t = float(np.median(times))
    return {"value": round(wl.kv_bytes / t / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "whole workload (%d query rows, %d keys), %d repetitions, median %.3f s"
                      % (wl.batch * wl.q_len * wl.num_heads_q, int(wl.cache_seqlens.sum()),
                         len(times), t)}


if __name__ == "__main__":
    main()
