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

Beside it: the roofline of the split kernel, the spread of single launches,
the read-only probes over the same bytes (the empirical ceiling), and the
float64 oracle timed on the host cores.

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
                    choices=["c1", "c2", "c3", "c4", "c5"],
                    help="c3: paged bf16 B32 Hq32/Hkv8 d128 L~1000 (default); "
                         "c4: B4 Hq32/Hkv4 L16384; c5: ragged fp16 B128 d64; "
                         "c1: dense fp16 Hq8/Hkv2 d64 kvLen512; "
                         "c2: dense fp16 MHA 32 heads qLen4 d128 (--kv-len)")
    ap.add_argument("--kv-len", type=int, default=4096, help="c2 only")
    ap.add_argument("--num-splits", type=int, default=0, help="0 = planner")
    ap.add_argument("--no-length-sum", action="store_true",
                    help="paged: do not give the planner the sum of the lengths")
    ap.add_argument("--pools", type=int, default=4, help="KV pool copies rotated over")
    ap.add_argument("--new-keys", type=int, default=0,
                    help="paged: each step appends this many keys a sequence in the same call "
                         "(attn_decode_kvcache_fwd; the last N keys of every sequence come "
                         "from k_new / v_new, holding the same values, so every step writes "
                         "the same bytes and attends the same keys)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the read-only probes (stream and page-gather reads of the "
                         "same KV bytes) that give the empirical ceiling")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, copy this many MiB device to device once (the "
                         "known-size copy that scales the HBM byte counters)")
    return ap.parse_args()


def make_workload(name, kv_len=4096):
    from split_kv_paged_amd import workloads as W
    if name == "c2":
        return W.c2_smallq(kv_len)
    return {"c1": W.c1_dense_decode, "c3": W.c3_paged_gqa4, "c4": W.c4_long,
            "c5": W.c5_ragged}[name]()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from split_kv_paged_amd import api

    wl = make_workload(args.workload, args.kv_len)
    dense = args.workload in ("c1", "c2")
    if dense and args.new_keys > 0:
        print("--new-keys appends to a paged cache: use a paged workload (c3, c4, c5)",
              file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[wl.dtype]

    def dev16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).to(dev)

    q = dev16(wl.q)
    stream = torch.cuda.current_stream(dev)
    out = torch.empty_like(q)
    # one prepared call per KV pool: the per-step host work is a single call
    # into the C ABI (which still plans and validates every time)
    if dense:
        pools = [(dev16(wl.k), dev16(wl.v)) for _ in range(max(1, args.pools))]
        lse = torch.empty((wl.num_heads_q, wl.q_len), dtype=torch.float32, device=dev)
        first = api.PreparedDense(q, pools[0][0], pools[0][1], num_splits=args.num_splits,
                                  softmax_scale=wl.scale, out=out, lse=lse, stream=stream)
        calls = [first] + [api.PreparedDense(q, k, v, num_splits=args.num_splits,
                                             softmax_scale=wl.scale, out=out, lse=lse,
                                             workspace=first.workspace, stream=stream)
                           for k, v in pools[1:]]
    else:
        pools = [(dev16(wl.k_cache), dev16(wl.v_cache)) for _ in range(max(1, args.pools))]
        bt = torch.from_numpy(wl.block_table).to(dev)
        sl = torch.from_numpy(wl.cache_seqlens).to(dev)
        lse = torch.empty((wl.batch, wl.num_heads_q, wl.q_len), dtype=torch.float32, device=dev)
        # a serving loop knows its lengths on the host; their sum lets the
        # planner split the longest sequences of a ragged batch
        hint = None if args.no_length_sum else int(wl.cache_seqlens.sum())
        kn = vn = None
        sl_call = sl
        if args.new_keys > 0:
            # the cache holds L_b - N keys before the call; the last N rows
            # of each sequence come in as k_new / v_new (the same values)
            N = args.new_keys
            if int(wl.cache_seqlens.min()) < N:
                print("--new-keys %d: a sequence of this workload has fewer keys" % N,
                      file=sys.stderr)
                sys.exit(2)
            old = (wl.cache_seqlens - N).astype(np.int32)
            shape = (wl.batch, N) + wl.k_cache.shape[2:]
            kb, vb = np.zeros(shape, np.uint16), np.zeros(shape, np.uint16)
            for b in range(wl.batch):
                for t in range(N):
                    pos = int(old[b]) + t
                    pg, slot = wl.block_table[b, pos // wl.page_size], pos % wl.page_size
                    kb[b, t], vb[b, t] = wl.k_cache[pg, slot], wl.v_cache[pg, slot]
            kn, vn = dev16(kb), dev16(vb)
            sl_call = torch.from_numpy(old).to(dev)
        first = api.PreparedDecode(q, pools[0][0], pools[0][1], bt, sl_call,
                                   num_splits=args.num_splits, softmax_scale=wl.scale,
                                   max_seqlen_k=wl.max_seqlen_k, out=out, lse=lse, stream=stream,
                                   sum_seqlen_k=hint, k_new=kn, v_new=vn)
        calls = [first] + [api.PreparedDecode(q, kc, vc, bt, sl_call,
                                              num_splits=args.num_splits,
                                              softmax_scale=wl.scale,
                                              max_seqlen_k=wl.max_seqlen_k, out=out, lse=lse,
                                              workspace=first.workspace, stream=stream,
                                              sum_seqlen_k=hint, k_new=kn, v_new=vn)
                           for kc, vc in pools[1:]]

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

    # Spread of single launches (outside the timed region): an event pair
    # around each of up to 100 launches.  The host then paces the launches,
    # so each starts on an idle GPU; the average above stays the figure.
    n_one = min(K, 100)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_one)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    one = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)

    def pct(q):
        return round(one[min(n_one - 1, int(q * (n_one - 1) + 0.5))], 3)

    ceiling = None
    if not args.no_ceiling:
        ceiling = read_ceiling(wl, pools, None if dense else (bt, sl),
                               last.split_keys if last.num_splits > 1 else 0, K, stream,
                               last.heads_per_row)

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
    batch = 1 if dense else wl.batch
    qheads = batch * wl.num_heads_q * wl.q_len
    if dense:
        config = {"workload": wl.name, "layout": "dense [H, len, d]", "num_heads_q":
                  wl.num_heads_q, "num_heads_kv": wl.num_heads_kv, "q_len": wl.q_len,
                  "kv_len": wl.kv_len, "head_dim": wl.head_dim}
    else:
        name = wl.name + ("_append%d" % args.new_keys if args.new_keys > 0 else "")
        config = {"workload": name, "batch": wl.batch, "q_len": wl.q_len,
                  "num_heads_q": wl.num_heads_q, "num_heads_kv": wl.num_heads_kv,
                  "head_dim": wl.head_dim, "page_size": wl.page_size,
                  "kv_tokens": int(wl.cache_seqlens.sum()),
                  "length_sum_given": not args.no_length_sum}
        if args.new_keys > 0:
            config.update({"new_keys": args.new_keys,
                           "appended_in_kernel": last.kernel >= 100000})
    config.update({"kv_bytes": kv_bytes, "num_splits": last.num_splits,
                   "pack_gqa": last.pack_gqa, "heads_per_row": last.heads_per_row,
                   "extra_blocks": last.extra_blocks, "grid": last.grid,
                   "kv_pools": len(pools), "accumulate": "f32"})

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
        "data": "synthetic (seeded N(0,1) %s Q/K/V%s)" % (
            wl.dtype, "" if dense else ", shuffled page table"),
        "config": config,
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "query_heads_per_s": round(qheads / wall, 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(config["workload"], last.num_splits),
            "kernel_avg_us": round(kern_s * 1e6, 3),
            "kernels_per_launch": 2 if args.new_keys > 0 and last.kernel < 100000 else 1,
        },
        "single_launch_us": {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9), "n": n_one,
                             "method": "event pair around each launch, host-paced"},
    }
    if ceiling is not None:
        ceiling["kernel_over_best_probe"] = round(
            achieved / max(v["GB/s"] for k, v in ceiling.items() if isinstance(v, dict)), 4)
        rec["read_ceiling"] = ceiling
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec), flush=True)


def read_ceiling(wl, pools, paged, split_keys, steps, stream, heads_per_row=1):
    """The empirical ceiling: read-only probes (libattn_probe.so) over the
    same KV bytes and pools as the timed calls, timed the same way (two
    events around `steps` back-to-back launches, pools rotated).
      stream_read       the first half of the KV bytes from each pool's K
                        tensor and the second half from its V tensor,
                        contiguous, one workgroup per compute unit
      page_gather_read  (paged) the valid keys' K and V rows, walked as the
                        decode kernel walks them (split as the timed calls
                        were, and with the calls' head groups read as one
                        wider row: the same bytes viewed as num_heads_kv / R
                        heads of R * head_dim), with no arithmetic"""
    import torch
    from split_kv_paged_amd import probe

    def timed(calls):
        for i in range(3):
            calls[i % len(calls)]()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            calls[i % len(calls)]()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    def entry(nbytes, us):
        gbs = nbytes / us / 1e3
        return {"GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4), "us": round(us, 3)}

    half = wl.kv_bytes // 2 // 16 * 16
    # one workgroup of 8 waves per compute unit: the fastest stream shape
    # measured (256 workgroups read these bytes in 19.8 us, 512 in 22.3)
    cus = torch.cuda.get_device_properties(pools[0][0].device).multi_processor_count
    sums = torch.empty(cus, dtype=torch.int32, device=pools[0][0].device)
    calls = [probe.prepared_stream_read(k, v, half, half, cus, sums, stream)[0] for k, v in pools]
    res = {"stream_read": entry(2 * half, timed(calls))}
    res["stream_read"]["workgroups"] = cus
    if paged is not None:
        bt, sl = paged
        R = max(1, heads_per_row)

        def view(t):  # R adjacent KV heads as one row of R * head_dim
            n, page, hkv, d = t.shape
            return t.view(n, page, hkv // R, R * d)
        first, psums = probe.prepared_page_read(view(pools[0][0]), view(pools[0][1]), bt, sl,
                                                wl.max_seqlen_k, split_keys, None, stream)
        calls = [first] + [probe.prepared_page_read(view(k), view(v), bt, sl, wl.max_seqlen_k,
                                                    split_keys, psums, stream)[0]
                           for k, v in pools[1:]]
        res["page_gather_read"] = entry(wl.kv_bytes, timed(calls))
        res["page_gather_read"]["split_keys"] = split_keys
        res["page_gather_read"]["heads_per_row"] = R
    res["method"] = "read-only probes over the same KV bytes and pools, events around %d " \
                    "back-to-back launches" % steps
    return res


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
    of repetitions (about budget_s seconds).  cores = the worker threads it
    used: every CPU the process may run on (nproc), at most the oracle's
    thread cap, one GPU's share of the measurement host."""
    import numpy as np

    import oracle
    threads = oracle.default_threads()
    dense = not hasattr(wl, "block_table")
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        if dense:
            oracle.dense_attention(wl.q, wl.k, wl.v, wl.dtype, scale=wl.scale, nthreads=threads)
        else:
            oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                   wl.cache_seqlens, wl.dtype, scale=wl.scale, nthreads=threads)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 20:
            break
    t = float(np.median(times))
    # one run on one thread, beside the all-threads median
    t1 = time.perf_counter()
    if dense:
        oracle.dense_attention(wl.q, wl.k, wl.v, wl.dtype, scale=wl.scale, nthreads=1)
    else:
        oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                               wl.cache_seqlens, wl.dtype, scale=wl.scale, nthreads=1)
    t1 = time.perf_counter() - t1
    rows = wl.q_len * wl.num_heads_q * (1 if dense else wl.batch)
    keys = wl.kv_len if dense else int(wl.cache_seqlens.sum())
    return {"value": round(wl.kv_bytes / t / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "whole workload (%d query rows, %d keys), %d repetitions, median %.3f s"
                      % (rows, keys, len(times), t),
            "single_thread_value": round(wl.kv_bytes / t1 / 1e9, 4),
            "nproc": oracle.host_cpus(), "host_threads": os.cpu_count(),
            "thread_cap": oracle.MAX_THREADS}


if __name__ == "__main__":
    main()
