"""Benchmark of the paged decode-attention hot path on one MI355X.

One step = one decode layer's attention step over a whole synthetic batch: every sequence
appends its current token (the KV-cache write of its K/V into its slot, fused into the split
pass of paged decode attention, which attends over the whole context including it), then the
merge pass.
The step reads every valid K/V byte of the batch once.  Steps rotate over --layers
separate pools (the same block tables, as the layers of one model would use), so no
pool is re-read before the others have streamed through; with 4 layers of the Llama-3-8B
batch that is ~2.6 GB between two reads of one pool, ten times the 256 MB MALL.

Printed on stdout: one JSON line.  value = KV GB/s of the whole step (algorithmic KV bytes
of valid tokens, sum_s L_s * Hkv * D * 2 * bytes, divided by the wall time per step);
roofline = the split kernel alone, timed in every fifth timed step by a pair of HIP events
that its own dispatch records (hipExtLaunchKernel) on its launch stream; the merge is timed
separately, after the timed region.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import statistics
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E peak (AMD public figure)
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (AMD public figure)
EVENT_EVERY = 5          # timed steps per sampled split-kernel duration
METRIC = "paged decode attention: KV GB/s (% HBM peak) and µs/step, Llama-3-8B shape"


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="llama3_8b_bf16")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--layers", type=int, default=4)
    p.add_argument("--num-splits", type=int, default=0)
    p.add_argument("--prefix-groups", choices=["on", "off"], default="on",
                   help="continuous batching over shared prefixes: read each group's shared blocks once for "
                        "all its sequences (on), or per sequence through the caches (off)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--traffic-json", default=None,
                   help="HBM traffic summary (default: profiles/paged_attention_split__<workload>__hbm_traffic.json)")
    p.add_argument("--op", choices=["kv_cache_write", "copy_blocks", "swap", "waste", "vmm"], default=None,
                   help="instead of the decode step, time one pool-maintenance kernel on the "
                        "workload's pool: the KV-cache write of the whole batch (the prefill "
                        "pattern) or copy_blocks of --pairs random block pairs")
    p.add_argument("--pairs", type=int, default=1024)
    p.add_argument("--vmm-page-kib", type=int, default=0,
                   help="--op vmm: page size in KiB of the virtual-memory pool (0: the paged pool)")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="instead of the benchmark, time plain device-to-device copies of MIB MiB "
                        "(the reference kernel for scaling the HBM byte counters)")
    return p.parse_args()


def _copy_probe(mib: int, reps: int = 10):
    """Plain copies of a known size: what FETCH_SIZE / WRITE_SIZE read for exactly `mib` MiB
    read and written calibrates the counters of the attention kernels."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    us = statistics.median(a.elapsed_time(b) for a, b in ev) * 1e3
    print(json.dumps({"probe": "device copy", "bytes_read": n, "bytes_written": n, "copies": reps,
                      "median_us": round(us, 2), "copy_GBps_read_plus_write": round(2 * n / us / 1e3, 1)}),
          flush=True)


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


TRAFFIC_UNIT = ("HBM bytes read + written per launch (rocprofv3 FETCH_SIZE, WRITE_SIZE, scaled by a plain copy "
                "of known size)")


def _set_blas_threads() -> int:
    """Gives the oracle's BLAS every core this process may run on; returns that count."""
    n = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(n)
    except Exception:  # pragma: no cover
        pass
    return n


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _traffic_from_profile(args, kernel: str, workload: str, files):
    """HBM bytes per launch from profiles/<kernel>__<workload>__hbm_traffic.json, reported only
    while the kernel sources it was taken on are the current ones."""
    path = args.traffic_json or os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                              f"{kernel}__{workload}__hbm_traffic.json")
    try:
        with open(path) as f:
            tj = json.load(f)
        if tj.get("workload") == workload and tj.get("kernel_source_sha") == _kernel_sha(files):
            return tj.get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        pass
    return None


def _cpu_baseline(case, bytes_per_token, budget_s=10.0, max_passes=3):
    """The oracle, as it stands, on the batch's sequences in a seeded random order, one at a
    time, until about `budget_s` of host time or `max_passes` passes over the batch.

    Returns (seconds, K/V bytes the oracle went through, sequences done, BLAS threads = the
    cores this process may run on)."""
    from oracle import attention as oatt
    blas_threads = _set_blas_threads()
    B = case.wl.batch
    order = np.random.default_rng(0).permutation(B)
    done_bytes, done_seqs = 0, 0
    t0 = time.perf_counter()
    for _ in range(max_passes):
        for sq in order.tolist():
            oatt.decode_case(case, [sq])
            done_bytes += int(case.lengths[sq]) * bytes_per_token
            done_seqs += 1
            if time.perf_counter() - t0 > budget_s:
                return time.perf_counter() - t0, done_bytes, done_seqs, blas_threads
    return time.perf_counter() - t0, done_bytes, done_seqs, blas_threads


def main():
    args = _args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the benchmark runs on one GPU only; multi-GPU runs are not supported "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        _copy_probe(args.copy_probe)
        return
    if args.op == "waste":
        _waste_report(args)
        return
    if args.op == "vmm":
        _vmm_bench(args)
        return
    if args.op:
        _op_bench(args)
        return

    import torch
    import paged_kv_cache_329_amd as pkv
    from synth import WORKLOADS, make_decode_case

    wl = WORKLOADS[args.workload]
    if wl.prefix_group:
        return _prefix_step_bench(args, wl)
    if wl.query_dist[0] != "one":
        return _multi_query_bench(args, wl)
    t0 = time.perf_counter()
    case = make_decode_case(wl, args.seed)
    _log(f"[bench] generated {wl.name} seed={args.seed} in {time.perf_counter() - t0:.1f}s; "
         f"sum L = {int(case.lengths.sum())}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kvt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3fn": torch.float8_e4m3fn}[wl.kv_dtype]
    eb = {"f32": 4, "bf16": 2, "fp8_e4m3fn": 1}[wl.kv_dtype]
    B, Hq, Hkv, D, bs = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size

    def dev_tensor(arr, storage):
        if storage == "f32":
            return torch.from_numpy(np.ascontiguousarray(arr, np.float32)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(arr, np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)

    store = "f32" if wl.kv_dtype == "f32" else "bf16"
    lens32 = case.lengths.astype(np.int32)
    t_meta = time.perf_counter()
    all_slots = pkv.build_slot_mapping(case.block_tables, lens32, bs)
    host_meta_us = (time.perf_counter() - t_meta) * 1e6
    k_tok, v_tok = dev_tensor(case.k, store), dev_tensor(case.v, store)
    slots_dev = torch.from_numpy(all_slots).to(dev)
    pools = []
    for _ in range(args.layers):
        k = pkv.allocate_kv_pool(case.num_blocks, Hkv, bs, D, kvt, dev)
        v = pkv.allocate_kv_pool(case.num_blocks, Hkv, bs, D, kvt, dev)
        pkv.kv_cache_write(k_tok, v_tok, k, v, slots_dev, k_scale=float(case.k_scale), v_scale=float(case.v_scale))
        pools.append((k, v))
    # The step's new tokens: each sequence's last token, appended again at position L-1
    # (its own slot) by every step.
    last = np.cumsum(case.lengths) - 1
    has = case.lengths > 0
    rows = torch.from_numpy(np.flatnonzero(has)).to(dev)
    src = torch.from_numpy(last[has]).to(dev)
    k_new = torch.zeros((B, Hkv, D), dtype=k_tok.dtype, device=dev)
    v_new = torch.zeros_like(k_new)
    k_new[rows] = k_tok.index_select(0, src)
    v_new[rows] = v_tok.index_select(0, src)
    del k_tok, v_tok, slots_dev
    q = dev_tensor(case.q, wl.q_dtype)
    out = torch.empty_like(q)
    tables = torch.from_numpy(case.block_tables).to(dev)
    lens = torch.from_numpy(lens32).to(dev)
    qd, kd = (pkv.F32 if wl.q_dtype == "f32" else pkv.BF16), {"f32": pkv.F32, "bf16": pkv.BF16,
                                                             "fp8_e4m3fn": pkv.FP8_E4M3FN}[wl.kv_dtype]
    ws_bytes = pkv.paged_attention_workspace_size(B, Hq, Hkv, D, bs, qd, kd, args.num_splits)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    splits = args.num_splits or pkv.paged_attention_default_splits(D, bs, qd, kd)
    stream = torch.cuda.current_stream(dev)
    ks, vs = float(case.k_scale), float(case.v_scale)

    def step(i, ev=None, detail=False):
        # One decode step: every sequence appends its token (stored into its slot by the
        # split pass itself) and attends over its whole context; then the merge pass.
        # ev: an event pair that the split kernel's own dispatch records at its start and
        # end (pkv_set_launch_events), so it times the kernel alone and adds no packets to
        # the stream; detail adds a stream event after the merge (used only outside the
        # timed region).
        k, v = pools[i % len(pools)]
        if ev is not None:
            pkv.set_launch_events(ev[0], ev[1])
        pkv.paged_decode_step_split(out, q, k_new, v_new, k, v, tables, lens, case.scale, ks, vs,
                                    args.num_splits, ws)
        pkv.paged_attention_reduce(out, q, k, v, tables, lens, case.scale, ks, vs, args.num_splits, ws)
        if detail:
            ev[2].record(stream)

    def new_events(n, per):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(per)] for _ in range(n)]
        for pair in evs:            # create them on the device before they are handed over
            for e in pair:
                e.record(stream)
        torch.cuda.synchronize()
        return evs

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # The split kernel is bracketed by events on every EVENT_EVERY-th timed step (5 is
    # coprime with the 4 layer pools, so the sample visits every pool).
    sampled = list(range(0, args.steps, EVENT_EVERY))
    events = dict(zip(sampled, new_events(len(sampled), 2)))
    _log(f"[bench] warmup done; timing {args.steps} steps over {len(pools)} layer pools")
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i, events.get(i))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    split_us = statistics.mean(e[0].elapsed_time(e[1]) for e in events.values()) * 1e3
    # Per-kernel breakdown, outside the timed region.
    n_detail = min(args.steps, 50)
    detail = new_events(n_detail, 3)
    for i in range(n_detail):
        step(i, detail[i], detail=True)
    torch.cuda.synchronize()
    merge_us = statistics.mean(e[1].elapsed_time(e[2]) for e in detail) * 1e3  # incl. the launch gap
    step_event_us = statistics.mean(e[0].elapsed_time(e[2]) for e in detail) * 1e3

    sum_l = int(case.lengths.sum())
    kv_bytes = sum_l * Hkv * D * 2 * eb
    us_per_step = elapsed / args.steps * 1e6
    value = kv_bytes / (us_per_step * 1e-6) / 1e9
    achieved = kv_bytes / (split_us * 1e-6) / 1e9

    traffic = _traffic_from_profile(args, "paged_attention_split", wl.name, ("attention_decode.hip", "attention_tile.h"))

    cpu = None
    if not args.no_cpu_baseline:
        _log("[bench] timing the fp64 oracle on the host (cpu_baseline)")
        t_cpu, cpu_bytes, cpu_seqs, threads = _cpu_baseline(case, Hkv * D * 2 * eb)
        cpu = {"value": round(cpu_bytes / t_cpu / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "cpu_model": _cpu_model(),
               "sample": f"{cpu_seqs} sequences of the batch ({B} sequences, sum L = {sum_l}) in a seeded random "
                         f"order, up to 3 passes or about 10 s: {cpu_bytes / 1e9:.3f} GB of K/V in {t_cpu:.2f} s, "
                         f"fp64 numpy oracle incl. decoding K/V to fp64"}

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_per_step / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8_e4m3fn": "fp8_e4m3fn+bf16"}[wl.kv_dtype],
        "data": "synthetic (seeded N(0,1) q/K/V, random physical block permutation)",
        "config": {"workload": wl.name, "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
                   "block_size": bs, "kv_dtype": wl.kv_dtype, "context": list(wl.length_dist),
                   "sum_context": sum_l, "num_blocks": case.num_blocks, "seed": args.seed,
                   "num_splits": int(splits), "layer_pools": len(pools)},
        "us_per_step": round(us_per_step, 2),
        "kv_bytes": kv_bytes,
        "hbm_frac": round(value / HBM_PEAK_GBPS, 4),
        "kernel_us": {"paged_attention_split(append)": round(split_us, 2),
                      "detail_outside_timed_region": {"paged_attention_merge": round(merge_us, 2),
                                                      "step_with_events": round(step_event_us, 2)}},
        "host_metadata_us": round(host_meta_us, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "traffic_unit": TRAFFIC_UNIT,
                     "algorithmic_bytes": kv_bytes, "kernel": "paged_attention_split_kernel (decode step with append)"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def _multi_query_bench(args, wl):
    """Causal multi-query attention (prefill, prefill chunk, drafted-token check): one step is
    one pkv_paged_attention_prefill call over the whole batch, on one of `layers` pools.

    Algorithmic work: every query at position P attends to P + 1 keys, 4 * D flops per key and
    query head (QK^T and PV), and every K/V byte of the batch is read at least once per kv
    head.  The roofline is the one the arithmetic intensity puts the workload under: MFMA
    (bf16, 2.5 PFLOP/s) above the ridge of 2.5e15 / 8e12 flop/B, HBM below it.
    """
    import torch
    import paged_kv_cache_329_amd as pkv
    from synth import make_prefill_case

    t0 = time.perf_counter()
    case = make_prefill_case(wl, args.seed)
    _log(f"[bench] generated {wl.name} seed={args.seed} in {time.perf_counter() - t0:.1f}s; "
         f"sum L = {int(case.lengths.sum())}, query tokens = {case.num_q_tokens}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kvt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3fn": torch.float8_e4m3fn}[wl.kv_dtype]
    eb = {"f32": 4, "bf16": 2, "fp8_e4m3fn": 1}[wl.kv_dtype]
    B, Hq, Hkv, D, bs = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size

    def dev_tensor(arr, storage):
        if storage == "f32":
            return torch.from_numpy(np.ascontiguousarray(arr, np.float32)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(arr, np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)

    store = "f32" if wl.kv_dtype == "f32" else "bf16"
    lens32 = case.lengths.astype(np.int32)
    slots_dev = torch.from_numpy(pkv.build_slot_mapping(case.block_tables, lens32, bs)).to(dev)
    k_tok, v_tok = dev_tensor(case.k, store), dev_tensor(case.v, store)
    pools = []
    for _ in range(args.layers):
        k = pkv.allocate_kv_pool(case.num_blocks, Hkv, bs, D, kvt, dev)
        v = pkv.allocate_kv_pool(case.num_blocks, Hkv, bs, D, kvt, dev)
        pkv.kv_cache_write(k_tok, v_tok, k, v, slots_dev, k_scale=float(case.k_scale), v_scale=float(case.v_scale))
        pools.append((k, v))
    del k_tok, v_tok, slots_dev
    q = dev_tensor(case.q, wl.q_dtype)
    out = torch.empty_like(q)
    tables = torch.from_numpy(case.block_tables).to(dev)
    lens = torch.from_numpy(lens32).to(dev)
    qstart = torch.from_numpy(case.query_start.astype(np.int32)).to(dev)
    max_q = int(case.q_lens.max())
    stream = torch.cuda.current_stream(dev)
    ks, vs = float(case.k_scale), float(case.v_scale)
    qd = pkv.F32 if wl.q_dtype == "f32" else pkv.BF16
    kd = {"f32": pkv.F32, "bf16": pkv.BF16, "fp8_e4m3fn": pkv.FP8_E4M3FN}[wl.kv_dtype]
    ws_bytes = pkv.paged_attention_prefill_workspace_size(B, Hq, Hkv, D, bs, qd, kd, max_q, args.num_splits)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    few = max_q * (Hq // Hkv) <= pkv.FEW_QUERY_COLUMNS
    path = ("split over keys + merge (few queries)" if few
            else "query tiles through LDS, launched longest first by a plan pass")

    def step(i, ev=None):
        k, v = pools[i % len(pools)]
        if ev is not None:
            pkv.set_launch_events(ev[0], ev[1])
        pkv.paged_attention_prefill(out, q, k, v, tables, lens, qstart, max_q, case.scale, ks, vs,
                                    num_splits=args.num_splits, workspace=ws)

    def new_events(n):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        for pair in evs:
            for e in pair:
                e.record(stream)
        torch.cuda.synchronize()
        return evs

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    sampled = list(range(0, args.steps, EVENT_EVERY))
    events = dict(zip(sampled, new_events(len(sampled))))
    _log(f"[bench] warmup done; timing {args.steps} steps over {len(pools)} layer pools")
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i, events.get(i))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    kernel_us = statistics.mean(e[0].elapsed_time(e[1]) for e in events.values()) * 1e3

    # Keys per query: P + 1 for P = L - n + i >= 0.
    keys = 0
    for L, n in zip(case.lengths.tolist(), case.q_lens.tolist()):
        first = L - n + 1                       # keys of query 0
        lo = max(first, 1)
        hi = L                                  # keys of the last query
        if hi >= lo:
            keys += (lo + hi) * (hi - lo + 1) // 2
    flops = keys * Hq * 4 * D
    sum_l = int(case.lengths.sum())
    kv_bytes = sum_l * Hkv * D * 2 * eb
    us_per_step = elapsed / args.steps * 1e6
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    mfma_bound = flops / kv_bytes > ridge
    if mfma_bound:
        metric, unit = "attention TFLOP/s", "TFLOP/s"
        value = flops / (us_per_step * 1e-6) / 1e12
        achieved = flops / (kernel_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                "algorithmic_flops": flops}
    else:
        metric, unit = "KV GB/s", "GB/s"
        value = kv_bytes / (us_per_step * 1e-6) / 1e9
        achieved = kv_bytes / (kernel_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None, "algorithmic_bytes": kv_bytes}
    roof["kernel"] = "paged_attention_mq_split_kernel" if few else "paged_attention_prefill_kernel"
    roof["path"] = path
    roof["traffic_unit"] = TRAFFIC_UNIT
    qb = 4 if wl.q_dtype == "f32" else 2
    roof["q_out_bytes"] = 2 * case.num_q_tokens * Hq * D * qb
    roof["traffic"] = _traffic_from_profile(args, "paged_attention_mq_split" if few else "paged_attention_prefill",
                                            wl.name, ("attention_prefill.hip", "attention_tile.h"))

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import attention as oatt
        _log("[bench] timing the fp64 oracle on the host (cpu_baseline)")
        threads = _set_blas_threads()
        # Query rows spread evenly over the batch, in chunks, until about 10 s of oracle work.
        order = np.linspace(0, case.num_q_tokens - 1, min(case.num_q_tokens, 16384)).astype(np.int64)
        order = order[np.random.default_rng(0).permutation(len(order))]   # every chunk spans the batch
        qs = case.query_start.astype(np.int64)
        done = []
        t_cpu0 = time.perf_counter()
        for c0 in range(0, len(order), 256):
            chunk = order[c0:c0 + 256]
            oatt.prefill_case(case, chunk)
            done.extend(chunk.tolist())
            if time.perf_counter() - t_cpu0 > 10.0:
                break
        t_cpu = time.perf_counter() - t_cpu0
        rows = np.array(done, dtype=np.int64)
        nrows = len(rows)
        sample_keys = 0
        for r in rows.tolist():
            s_ = int(np.searchsorted(qs, r, side="right") - 1)
            P = int(case.lengths[s_]) - int(case.q_lens[s_]) + (r - int(qs[s_]))
            sample_keys += max(P + 1, 0)
        sflops = sample_keys * Hq * 4 * D
        if mfma_bound:
            cval, cunit = sflops / t_cpu / 1e12, "TFLOP/s"
        else:
            # The sample's share of the batch's work, in the metric's bytes.
            cval, cunit = kv_bytes * (sample_keys / max(keys, 1)) / t_cpu / 1e9, "GB/s"
        cpu = {"value": round(cval, 6), "unit": cunit, "cores": threads, "kind": "oracle",
               "cpu_model": _cpu_model(),
               "sample": f"{nrows} query rows drawn evenly over the batch ({sample_keys} keys in all, about 10 s), "
                         f"fp64 numpy oracle incl. decoding each touched sequence's K/V to fp64, {t_cpu:.1f} s"}

    result = {
        "metric": metric,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_per_step / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8_e4m3fn": "fp8_e4m3fn+bf16"}[wl.kv_dtype],
        "data": "synthetic (seeded N(0,1) q/K/V, random physical block permutation)",
        "config": {"workload": wl.name, "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
                   "block_size": bs, "kv_dtype": wl.kv_dtype, "context": list(wl.length_dist),
                   "queries": list(wl.query_dist), "sum_context": sum_l, "query_tokens": case.num_q_tokens,
                   "num_blocks": case.num_blocks, "seed": args.seed, "layer_pools": len(pools)},
        "us_per_step": round(us_per_step, 2),
        "flops": flops,
        "kv_bytes": kv_bytes,
        "kernel_us": {"paged_attention_prefill": round(kernel_us, 2)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def _waste_report(args):
    """Allocation waste and capacity on the synthetic length distributions (host only).

    For each workload's drawn lengths: the share of allocated KV slots that hold no token under
    paging with blocks of 16 and 32 (the real allocator, pkv_alloc_stats_get) and under a
    contiguous reservation of the distribution's maximum length per sequence; and how many
    sequences drawn from the same distribution fit in a fixed budget (the paged pool the
    workload sizes at 16-token blocks) either way.  For the prefix-sharing workload the
    allocator also forks each group from its root, and shared blocks count once.
    """
    import paged_kv_cache_329_amd as pkv
    from synth import WORKLOADS, draw_lengths

    names = [args.workload] if args.workload != "llama3_8b_bf16" else \
        ["llama3_8b_bf16", "cont_batch_prefix_bf16", "long_ctx_splitk_bf16", "fp8_kv"]
    for name in names:
        wl = WORKLOADS[name]
        rng = np.random.default_rng(np.random.SeedSequence(args.seed).spawn(6)[0])
        lengths = draw_lengths(wl, rng)
        max_len = int(wl.length_dist[2] if wl.length_dist[0] == "uniform" else wl.length_dist[3])
        if wl.prefix_group:
            max_len = max(max_len, wl.prefix_len)
        row = {"op": "waste", "workload": name, "sequences": int(len(lengths)), "sum_tokens": int(lengths.sum()),
               "max_len": max_len}
        budget_slots = None
        for bs in (16, 32):
            need = int(sum((int(L) + bs - 1) // bs for L in lengths))
            groups = wl.batch // wl.prefix_group if wl.prefix_group else 0
            nb = need + groups * ((wl.prefix_len + bs - 1) // bs) + 1
            a = pkv.BlockAllocator(nb, bs)
            if groups:
                for gi in range(groups):
                    a.seq_create(1_000_000 + gi, wl.prefix_len)
                for i, L in enumerate(lengths.tolist()):
                    root = 1_000_000 + i // wl.prefix_group
                    a.fork(root, i, min(L, wl.prefix_len))
                    if L > wl.prefix_len:
                        a.extend(i, L - wl.prefix_len)
                for gi in range(groups):
                    a.free(1_000_000 + gi)
            else:
                for i, L in enumerate(lengths.tolist()):
                    a.seq_create(i, L)
            st = a.stats()
            a.close()
            held = st["used_blocks"] * bs
            row[f"paged_bs{bs}"] = {"blocks_used": st["used_blocks"], "shared_blocks": st["shared_blocks"],
                                    "logical_blocks": st["logical_blocks"], "slots_held": held,
                                    "stored_tokens": st["stored_tokens"],
                                    "waste_frac": round(1 - st["stored_tokens"] / held, 5)}
            if bs == 16:
                budget_slots = int(math.ceil(1.1 * held))
        row["contiguous_max_len"] = {"slots_held": int(len(lengths)) * max_len,
                                     "waste_frac": round(1 - int(lengths.sum()) / (len(lengths) * max_len), 5)}
        # Capacity in the same budget: sequences from the same distribution until one does not fit.
        cap_rng = np.random.default_rng(args.seed + 1)
        more = draw_lengths(wl.scaled(batch=200_000), cap_rng)
        fits_paged, used = 0, 0
        for L in more.tolist():
            blocks = (L + 15) // 16
            if used + blocks * 16 > budget_slots:
                break
            used += blocks * 16
            fits_paged += 1
        row["budget_slots"] = budget_slots
        row["sequences_that_fit"] = {"paged_bs16": fits_paged, "contiguous_max_len": budget_slots // max_len}
        print(json.dumps(row), flush=True)


def _vmm_bench(args):
    """Decode over the same K/V in several placements: the paged pool with blocks in random
    order, each sequence's blocks consecutive in an ordinary pool, and contiguous per-sequence
    slices of virtual memory mapped on demand (pkv_vmm_*) with --vmm-page-kib pages (one
    placement per process).  Contiguous placements are read both by the paged kernel through
    a table counting up from each sequence's first block and by the contiguous kernel, which
    computes the addresses.  Each uses --layers copies so that a step reads from HBM; the split
    kernel is timed by its dispatch-recorded events on every step."""
    import torch
    import paged_kv_cache_329_amd as pkv
    from synth import WORKLOADS, make_decode_case

    wl = WORKLOADS[args.workload]
    if wl.prefix_group or wl.kv_dtype != "bf16":
        raise SystemExit("--op vmm runs on the bf16 decode workloads")
    case = make_decode_case(wl, args.seed)
    dev = torch.device("cuda:0")
    B, Hq, Hkv, D, bs = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size
    lens32 = case.lengths.astype(np.int32)
    nbs = [(int(L) + bs - 1) // bs for L in case.lengths]
    max_blocks = max(1, max(nbs))
    kt = torch.from_numpy(np.ascontiguousarray(case.k, np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)
    vt = torch.from_numpy(np.ascontiguousarray(case.v, np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)
    q = torch.from_numpy(np.ascontiguousarray(case.q, np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)
    out = torch.empty_like(q)
    lens = torch.from_numpy(lens32).to(dev)
    kv_bytes = int(case.lengths.sum()) * Hkv * D * 2 * 2
    layouts, failed = {}, {}
    if args.vmm_page_kib == 0:
        paged = []
        ptab = torch.from_numpy(case.block_tables).to(dev)
        pslots = torch.from_numpy(pkv.build_slot_mapping(case.block_tables, lens32, bs)).to(dev)
        for _ in range(args.layers):
            k = pkv.allocate_kv_pool(case.num_blocks, Hkv, bs, D, torch.bfloat16, dev)
            v = pkv.allocate_kv_pool(case.num_blocks, Hkv, bs, D, torch.bfloat16, dev)
            pkv.kv_cache_write(kt, vt, k, v, pslots)
            paged.append((k, v, ptab))
        layouts["paged_random_blocks"] = (paged, case.num_blocks * Hkv * bs * D * 2 * 2 * args.layers, None)
        # The same K/V with each sequence's blocks consecutive in an ordinary pool.
        first = np.concatenate([[0], np.cumsum(nbs)[:-1]]).astype(np.int32)
        ctab = np.full((B, max_blocks), -1, dtype=np.int32)
        for s_, nb in enumerate(nbs):
            ctab[s_, :nb] = first[s_] + np.arange(nb)
        cslots = torch.from_numpy(pkv.build_slot_mapping(ctab, lens32, bs)).to(dev)
        contig = []
        for _ in range(args.layers):
            k = pkv.allocate_kv_pool(int(sum(nbs)), Hkv, bs, D, torch.bfloat16, dev)
            v = pkv.allocate_kv_pool(int(sum(nbs)), Hkv, bs, D, torch.bfloat16, dev)
            pkv.kv_cache_write(kt, vt, k, v, cslots)
            contig.append((k, v, torch.from_numpy(ctab).to(dev), None, torch.from_numpy(first).to(dev)))
        layouts["contiguous_in_pool"] = (contig, int(sum(nbs)) * Hkv * bs * D * 2 * 2 * args.layers, None)
    else:
        page = args.vmm_page_kib << 10
        name = f"vmm_{args.vmm_page_kib}KiB_pages"
        pools, mapped = [], 0
        t0 = time.perf_counter()
        n_pages = 0
        try:
            for _ in range(args.layers):
                vmm = pkv.VmmPool(B, max_blocks, Hkv, bs, D, torch.bfloat16, page_bytes=page)
                pools.append((vmm.k, vmm.v, None, vmm))
                tables = np.full((B, max_blocks), -1, dtype=np.int32)
                for s_, nb in enumerate(nbs):
                    vmm.reserve(s_, nb)
                    tables[s_, :nb] = vmm.first_block(s_) + np.arange(nb)
                n_pages += (vmm.mapped_bytes // vmm.page_bytes) - 2
                firsts = torch.tensor([vmm.first_block(s_) for s_ in range(B)], dtype=torch.int32, device=dev)
                pools[-1] = (vmm.k, vmm.v, torch.from_numpy(tables).to(dev), vmm, firsts)
                mapped += vmm.mapped_bytes
        except pkv.PagedKVError as e:
            # Record how far the mapping got: the GPU kernel driver caps the number of allocations.
            last = pools[-1][3] if pools else None
            if last is not None and pools[-1][2] is None:
                n_pages += (last.mapped_bytes // last.page_bytes) - 2
            failed[name] = {"page_bytes": page, "error": str(e), "pages_mapped_before_failure": int(n_pages)}
            for p_ in pools:
                p_[3].close()
            pools = []
        if pools:
            map_s = time.perf_counter() - t0
            for k, v, t, _, _ in pools:
                slots = torch.from_numpy(pkv.build_slot_mapping(t.cpu().numpy(), lens32, bs)).to(dev)
                pkv.kv_cache_write(kt, vt, k, v, slots)
            layouts[name] = (pools, mapped, {"page_bytes": pools[0][3].page_bytes,
                                             "map_us_per_page": round(map_s * 1e6 / max(1, n_pages), 2),
                                             "pages_mapped": int(n_pages)})
    del kt, vt
    qd, kd = pkv.BF16, pkv.BF16
    ws = torch.empty(pkv.paged_attention_workspace_size(B, Hq, Hkv, D, bs, qd, kd, 0), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    rows = {}
    runs = [(name, entry, False) for name, entry in layouts.items()]
    # Contiguous placements are also read by the contiguous kernel (addresses computed from each
    # sequence's first block, no table loads).
    runs += [(name + "+contiguous_kernel", entry, True) for name, entry in layouts.items()
             if len(entry[0][0]) > 4]
    for name, (pools, mapped, extra), contiguous in runs:
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for pair in evs:
            for e in pair:
                e.record(stream)
        torch.cuda.synchronize()
        for i in range(args.warmup + args.steps):
            entry = pools[i % len(pools)]
            k, v, t = entry[:3]
            if i >= args.warmup:
                pkv.set_launch_events(*evs[i - args.warmup])
            if contiguous:
                pkv.contiguous_attention_decode(out, q, k, v, entry[4], lens, t.shape[1], case.scale, workspace=ws)
            else:
                pkv.paged_attention_decode(out, q, k, v, t, lens, case.scale, num_splits=0, workspace=ws)
        torch.cuda.synchronize()
        us = statistics.mean(e[0].elapsed_time(e[1]) for e in evs) * 1e3
        rows[name] = {"split_kernel_us": round(us, 2), "GBps": round(kv_bytes / (us * 1e-6) / 1e9, 1),
                      "device_bytes_backing_kv": int(mapped),
                      "kernel": "contiguous (computed addresses)" if contiguous else "paged (block table)"}
        if extra:
            rows[name].update(extra)
    print(json.dumps({"op": "vmm", "workload": wl.name, "kv_bytes": kv_bytes, "layers": args.layers,
                      "layouts": rows, "could_not_map": failed}), flush=True)
    for pools, _, _ in layouts.values():
        for entry in pools:
            if len(entry) > 3 and entry[3] is not None:
                entry[3].close()


def _op_bench(args):
    """Bandwidth of one pool-maintenance kernel (its own JSON line, not the headline)."""
    import torch
    import paged_kv_cache_329_amd as pkv
    from synth import WORKLOADS, make_decode_case

    wl = WORKLOADS[args.workload]
    if wl.prefix_group:
        raise SystemExit("--op runs on the decode workloads")
    case = make_decode_case(wl, args.seed)
    dev = torch.device("cuda:0")
    kvt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8_e4m3fn": torch.float8_e4m3fn}[wl.kv_dtype]
    eb = {"f32": 4, "bf16": 2, "fp8_e4m3fn": 1}[wl.kv_dtype]
    inb = 4 if wl.kv_dtype == "f32" else 2
    Hkv, D, bs = wl.num_kv_heads, wl.head_dim, wl.block_size
    pools = [(pkv.allocate_kv_pool(case.num_blocks, Hkv, bs, D, kvt, dev),
              pkv.allocate_kv_pool(case.num_blocks, Hkv, bs, D, kvt, dev)) for _ in range(max(1, args.layers))]

    def dev_tensor(arr):
        if wl.kv_dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(arr, np.float32)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(arr, np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)

    ks, vs = float(case.k_scale), float(case.v_scale)
    if args.op == "kv_cache_write":
        slots = torch.from_numpy(pkv.build_slot_mapping(case.block_tables, case.lengths.astype(np.int32), bs)).to(dev)
        kt, vt = dev_tensor(case.k), dev_tensor(case.v)
        T = int(slots.numel())
        nbytes = T * Hkv * D * 2 * (inb + eb)           # read K, V in; write K, V out

        def run(i):
            k, v = pools[i % len(pools)]
            pkv.kv_cache_write(kt, vt, k, v, slots, k_scale=ks, v_scale=vs)
        what = f"{T} tokens x {Hkv} kv heads into their slots (prefill pattern)"
    elif args.op == "copy_blocks":
        rng = np.random.default_rng(args.seed)
        ids = rng.permutation(case.num_blocks)
        n = min(args.pairs, case.num_blocks // 2)
        pairs = torch.from_numpy(np.stack([ids[:n], ids[n:2 * n]], 1).astype(np.int32)).to(dev)
        nbytes = n * 2 * Hkv * bs * D * eb * 2          # K and V blocks, read + write

        def run(i):
            k, v = pools[i % len(pools)]
            pkv.copy_blocks(k, v, pairs, D)
        what = f"{n} random (src, dst) block pairs, whole blocks of K and V"
    if args.op == "swap":
        return _swap_bench(args, wl, case, pools[0], kvt, eb)
    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    gbps = nbytes / (us * 1e-6) / 1e9
    print(json.dumps({"op": args.op, "workload": wl.name, "what": what, "us_per_call": round(us, 2),
                      "bytes_read_plus_written": int(nbytes), "GBps": round(gbps, 1),
                      "frac_of_8TBps": round(gbps / HBM_PEAK_GBPS, 4)}), flush=True)


def _swap_bench(args, wl, case, pool, kvt, eb):
    """Swap-out (device pool -> pinned host pool) and swap-in (back into other device blocks)
    of --pairs random blocks with pkv_swap_blocks, against torch's contiguous copy of the same
    number of bytes between device memory and pinned host memory."""
    import torch
    import paged_kv_cache_329_amd as pkv

    dev = torch.device("cuda:0")
    k, v = pool
    Hkv, D, bs = wl.num_kv_heads, wl.head_dim, wl.block_size
    n = min(args.pairs, case.num_blocks // 2)
    rng = np.random.default_rng(args.seed)
    ids = rng.permutation(case.num_blocks)
    hk = pkv.allocate_host_pool(n, Hkv, bs, D, kvt)
    hv = pkv.allocate_host_pool(n, Hkv, bs, D, kvt)
    out_pairs = torch.from_numpy(np.stack([ids[:n], np.arange(n)], 1).astype(np.int32)).to(dev)
    in_pairs = torch.from_numpy(np.stack([np.arange(n), ids[n:2 * n]], 1).astype(np.int32)).to(dev)
    nbytes = n * 2 * Hkv * bs * D * eb                  # K and V blocks moved one way
    flat_d = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    flat_h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps

    # The same scattered swap done by the copy engines instead: one hipMemcpyAsync per block
    # of K and per block of V, issued from the host on torch's stream (the runtime already
    # loaded in this process, found by its mapped path).
    hip = _loaded_hip_runtime()
    blk = Hkv * bs * D * eb                              # one block of K (or of V), bytes
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out_np, in_np = out_pairs.cpu().numpy(), in_pairs.cpu().numpy()

    def dma(dk, dv, sk, sv, pairs):
        for src, dst in pairs.tolist():
            for d_t, s_t in ((dk, sk), (dv, sv)):
                rc = hip.hipMemcpyAsync(ctypes.c_void_p(d_t.data_ptr() + dst * blk),
                                        ctypes.c_void_p(s_t.data_ptr() + src * blk), ctypes.c_size_t(blk),
                                        4, stream)   # hipMemcpyDefault: direction from the pointers
                if rc != 0:
                    raise RuntimeError(f"hipMemcpyAsync failed with code {rc}")

    res = {"out": timed(lambda: pkv.swap_blocks(hk, hv, k, v, out_pairs, D)),
           "in": timed(lambda: pkv.swap_blocks(k, v, hk, hv, in_pairs, D)),
           "dma_out": timed(lambda: dma(hk, hv, k, v, out_np)),
           "dma_in": timed(lambda: dma(k, v, hk, hv, in_np)),
           "copy_d2h": timed(lambda: flat_h.copy_(flat_d, non_blocking=True)),
           "copy_h2d": timed(lambda: flat_d.copy_(flat_h, non_blocking=True))}
    gb = {key: round(nbytes / (us * 1e-6) / 1e9, 2) for key, us in res.items()}
    print(json.dumps({"op": "swap", "workload": wl.name,
                      "what": f"{n} random blocks (K and V, {nbytes} bytes) device -> pinned host and back",
                      "dma": "dma_out / dma_in: the same pairs as 2n hipMemcpyAsync calls (one per block of K and of V)",
                      "us_per_call": {key: round(us, 2) for key, us in res.items()}, "bytes_one_way": nbytes,
                      "GBps": gb}), flush=True)


def _loaded_hip_runtime():
    """The HIP runtime library this process has already loaded (torch's), via its mapped path."""
    with open("/proc/self/maps") as f:
        paths = {line.split()[-1] for line in f if "libamdhip64.so" in line}
    if not paths:
        raise RuntimeError("no HIP runtime is loaded in this process")
    hip = ctypes.CDLL(sorted(paths)[0])
    hip.hipMemcpyAsync.restype = ctypes.c_int
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    return hip


def _prefix_step_bench(args, wl):
    """Continuous-batching steps over prefix-sharing groups (one pool; timed steps follow
    one another, each appending one token to every sequence).

    A step: the C++ allocator appends a token to every sequence (slots, and copy-on-write
    pairs for shared partial tails) into a pinned host buffer; only the slots (and pairs) go
    to the device, asynchronously; then copy_blocks, pkv_apply_append (the device copies of
    the block tables and lengths take the step's change), the decode step (the KV write of
    each token fused into the split pass) and the merge.  Host buffers are double-buffered
    so the host prepares step i+1 while the GPU runs step i.  pkv_apply_append reads the
    slots straight from the pinned host buffer; only copy-on-write pairs (the first step's)
    are uploaded.
    """
    import math

    import torch
    import paged_kv_cache_329_amd as pkv
    from paged_kv_cache_329_amd.step import DecodeStep
    from synth import make_prefix_step_case

    t0 = time.perf_counter()
    case = make_prefix_step_case(wl, args.seed)
    _log(f"[bench] generated {wl.name} seed={args.seed} in {time.perf_counter() - t0:.1f}s; "
         f"sum L = {int(case.lengths.sum())}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, Hq, Hkv, D, bs, P = (wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size,
                            wl.prefix_len)
    n_steps = args.warmup + args.steps
    # Room for every step's appends on top of the workload's pool.
    extra = B * ((n_steps + 20) // bs + 2)
    nb = case.num_blocks + extra
    order = np.concatenate([case.free_order, np.arange(case.num_blocks, nb, dtype=np.int32)])

    def bf16(arr):
        return torch.from_numpy(np.ascontiguousarray(arr, np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)

    a = pkv.BlockAllocator(nb, bs, free_order=order)
    k = pkv.allocate_kv_pool(nb, Hkv, bs, D, torch.bfloat16, dev)
    v = pkv.allocate_kv_pool(nb, Hkv, bs, D, torch.bfloat16, dev)
    root = 1 << 40
    for g in range(case.groups):
        slots = a.seq_create(root + g, P)
        pkv.kv_cache_write(bf16(case.root_k[g]), bf16(case.root_v[g]), k, v, torch.from_numpy(slots).to(dev))
    priv = []
    for i in range(B):
        L = int(case.lengths[i])
        a.fork(root + i // wl.prefix_group, i, min(L, P))
        if L > P:
            priv.append(a.extend(i, L - P)[0])
    if priv:
        pkv.kv_cache_write(bf16(case.priv_k), bf16(case.priv_v), k, v,
                           torch.from_numpy(np.concatenate(priv)).to(dev))
    members = np.arange(B, dtype=np.int64)
    max_blocks = int(math.ceil((int(case.lengths.max()) + n_steps + 21) / bs))
    k_new, v_new, q = bf16(case.new_k), bf16(case.new_v), bf16(case.q)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)
    # With prefix groups each group's shared blocks are read once, for all its sequences, in
    # the same launch as every sequence's own blocks.  Without them, each sequence's shared
    # leading blocks go through the caches, and then twice the default split count measured
    # faster on MI355X: shorter shares bring the members of a group to a shared block closer
    # together in time, so more of their repeated reads hit in L2 or the MALL.
    groups_on = args.prefix_groups == "on"
    default = pkv.paged_attention_default_splits(D, bs, pkv.BF16, pkv.BF16)
    nsplits = args.num_splits or (default if groups_on else 2 * default)
    stepper = DecodeStep(a, members, k, v, D, Hq, max_blocks, num_splits=nsplits, shared_prefix=True,
                         prefix_groups=groups_on)
    prefix_counts = stepper.shared_counts
    shared = stepper.shared
    ws = stepper.ws
    lens_host = stepper.lens.cpu().numpy().astype(np.int64)
    host_s = [0.0]
    logical_bytes = []
    cows_seen = []

    def step(i, ev=None, after_copy=None):
        h0 = stepper.host_alloc_s
        n_cow = stepper.run(out, q, k_new, v_new, case.scale, kernel_events=ev, after_upload=after_copy)
        host_s[0] += stepper.host_alloc_s - h0
        cows_seen.append(n_cow)
        lens_host[:] += 1
        logical_bytes.append(int(lens_host.sum()) * Hkv * D * 2 * 2)

    # Load every kernel of the step once on a scratch pool, so that the first step's
    # timing (the one that copies every shared partial tail) holds no first-launch cost.
    sk = pkv.allocate_kv_pool(4, Hkv, bs, D, torch.bfloat16, dev)
    sv = torch.zeros_like(sk)
    sk.zero_()
    one = torch.ones(B, dtype=torch.int32, device=dev)
    st = torch.zeros((B, 1), dtype=torch.int32, device=dev)
    pkv.copy_blocks(sk, sv, torch.tensor([[0, 1]], dtype=torch.int32, device=dev), D)
    pkv.apply_append(torch.zeros((1, 1), dtype=torch.int32, device=dev), torch.zeros(1, dtype=torch.int32, device=dev),
                     torch.full((1,), -1, dtype=torch.int64, device=dev), bs, 4)
    if groups_on:
        zeros = torch.zeros(B, dtype=torch.int32, device=dev)
        pkv.paged_decode_step_grouped(out, q, k_new, v_new, sk, sv, st, one, (zeros, zeros, zeros), case.scale,
                                      num_splits=nsplits)
    else:
        pkv.paged_decode_step_split(out, q, k_new, v_new, sk, sv, st, one, case.scale, num_splits=nsplits,
                                    workspace=ws, shared_prefix_blocks=shared)
        pkv.paged_attention_reduce(out, q, sk, sv, st, one, case.scale, num_splits=nsplits, workspace=ws,
                                   shared_prefix_blocks=shared)
    del sk, sv, one, st
    # The first step copies every shared partial tail; time it on its own.
    e_first = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in e_first:
        e.record(stream)
    torch.cuda.synchronize()
    step(0, after_copy=e_first[0])             # GPU time from the metadata copies' end
    e_first[1].record(stream)
    torch.cuda.synchronize()
    first_us = e_first[0].elapsed_time(e_first[1]) * 1e3
    first_cow = cows_seen[0]
    for i in range(1, args.warmup):
        step(i)
    torch.cuda.synchronize()
    sampled = list(range(0, args.steps, EVENT_EVERY))
    events = {j: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for j in sampled}
    for pair in events.values():
        for e in pair:
            e.record(stream)
    torch.cuda.synchronize()
    host_s[0] = 0.0
    logical_bytes.clear()
    t_start = time.perf_counter()
    for j in range(args.steps):
        step(args.warmup + j, events.get(j))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    split_us = statistics.mean(e[0].elapsed_time(e[1]) for e in events.values()) * 1e3
    us_per_step = elapsed / args.steps * 1e6
    kv_bytes = statistics.mean(logical_bytes)
    # Where a step's GPU time goes (outside the timed region): stream events after the
    # host-to-device metadata copies and after the merge, the split kernel by its dispatch.
    n_detail = min(args.steps, 20)
    det = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_detail)]
    for d in det:
        for e in d:
            e.record(stream)
    torch.cuda.synchronize()
    for j in range(n_detail):
        d = det[j]
        d[0].record(stream)
        step(n_steps + j, (d[2], d[3]), d[1])
        d[4].record(stream)
    torch.cuda.synchronize()
    h2d_us = statistics.mean(d[0].elapsed_time(d[1]) for d in det) * 1e3
    to_split_us = statistics.mean(d[1].elapsed_time(d[2]) for d in det) * 1e3
    merge_us = statistics.mean(d[3].elapsed_time(d[4]) for d in det) * 1e3
    gpu_step_us = statistics.mean(d[0].elapsed_time(d[4]) for d in det) * 1e3
    # Unique physical KV bytes of the last step: each referenced block once, with the
    # largest number of valid tokens any referencing sequence reads in it.
    tables, lens = a.block_tables(members, max_blocks)
    lens = lens.astype(np.int64)
    assert np.array_equal(tables, stepper.tables.cpu().numpy())
    assert np.array_equal(lens, stepper.lens.cpu().numpy().astype(np.int64))
    used = {}
    for si in range(B):
        for j in range(int(math.ceil(lens[si] / bs))):
            b = int(tables[si, j])
            used[b] = max(used.get(b, 0), min(bs, int(lens[si]) - j * bs))
    unique_last = sum(used.values()) * Hkv * D * 2 * 2
    # Every step appends one private token per sequence, so the distinct bytes grow by exactly
    # B tokens per step: their mean over the timed steps is the last state's less the growth
    # since the middle of the timed region (the detail steps ran after it).
    unique_bytes = unique_last - B * Hkv * D * 2 * 2 * (n_detail + (args.steps - 1) / 2)
    value = kv_bytes / (us_per_step * 1e-6) / 1e9
    # The split kernel reads every distinct block once from HBM at best (shared prefix blocks
    # re-read by other members can come from L2 or the MALL): its roofline is on distinct bytes.
    achieved = unique_bytes / (split_us * 1e-6) / 1e9
    traffic = _traffic_from_profile(args, "paged_decode_step", wl.name, ("attention_decode.hip", "attention_tile.h"))

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import attention as oatt
        _log("[bench] timing the fp64 oracle on the host (cpu_baseline)")
        threads = _set_blas_threads()
        order = np.random.default_rng(0).permutation(B)
        done_bytes, done = 0, 0
        t_cpu0 = time.perf_counter()
        for sq in order.tolist():
            oatt.prefix_step_case(case, [sq])
            done_bytes += (int(case.lengths[sq]) + 1) * Hkv * D * 2 * 2
            done += 1
            if time.perf_counter() - t_cpu0 > 10.0:
                break
        t_cpu = time.perf_counter() - t_cpu0
        cpu = {"value": round(done_bytes / t_cpu / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "cpu_model": _cpu_model(),
               "sample": f"{done} of the {B} sequences in a seeded random order (about 10 s): their logical K/V "
                         f"after the step's append, {done_bytes / 1e9:.3f} GB in {t_cpu:.2f} s, fp64 numpy oracle "
                         f"incl. decoding K/V to fp64"}
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us_per_step / 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/K/V; groups of 8 share a live 1024-token root prefix)",
        "config": {"workload": wl.name, "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D,
                   "block_size": bs, "context": list(wl.length_dist), "prefix_group": wl.prefix_group,
                   "prefix_len": P, "seed": args.seed, "num_blocks": nb, "num_splits": int(nsplits)},
        "value_note": "value = logical KV bytes (every sequence's tokens, shared prefix blocks once per reader) "
                      "per wall-clock step",
        "us_per_step": round(us_per_step, 2),
        "kv_bytes_logical": int(kv_bytes),
        "kv_bytes_unique": int(unique_bytes),
        "kv_bytes_unique_note": "mean over the timed steps of the distinct K/V bytes (each physical block once, with "
                                "the most tokens any reader uses in it); logical = mean of every sequence's tokens",
        "unique_GBps": round(unique_bytes / (us_per_step * 1e-6) / 1e9, 2),
        "hbm_frac_unique": round(unique_bytes / (us_per_step * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "kernel_us": {"paged_attention_split(append)": round(split_us, 2),
                      "detail_outside_timed_region": {
                          "pair_upload": round(h2d_us, 2),
                          "to_split_start": round(to_split_us, 2),
                          "merge_incl_gap": round(merge_us, 2),
                          "gpu_step": round(gpu_step_us, 2)}},
        "host_allocator_us_per_step": round(host_s[0] / args.steps * 1e6, 1),
        "kv_loads": ("each group's shared blocks read once for all its sequences (prefix groups), non-temporal"
                     if groups_on else
                     "cached for each sequence's shared leading blocks, non-temporal for the rest"
                     if shared is not None else "non-temporal"),
        "shared_leading_blocks": int(prefix_counts.sum()),
        "first_step": {"copy_on_write_pairs": int(first_cow),
                       "gpu_us_copy_blocks_to_merge_end": round(first_us, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "traffic_unit": TRAFFIC_UNIT,
                     "algorithmic_bytes": int(unique_bytes),
                     "algorithmic_bytes_note": "distinct K/V bytes of a timed step, mean (each physical block once, "
                                               "with the most tokens any reader uses in it)",
                     "logical_GBps": round(kv_bytes / (split_us * 1e-6) / 1e9, 1),
                     "kernel": ("paged_attention_grouped_kernel (decode step with append, prefix groups)"
                                if groups_on else "paged_attention_split_kernel (decode step with append)")},
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


def _kernel_sha(files=("attention_decode.hip", "attention_tile.h")) -> str:
    """Hash of the sources a profiled kernel is built from (traffic figures are reported
    only while it matches)."""
    import hashlib
    h = hashlib.sha256()
    for name in files:
        p = os.path.join(os.path.dirname(os.path.abspath(__file__)), "paged_kv_cache_329_amd", "csrc", name)
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
