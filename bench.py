"""Benchmark of one paged decode step (or one prefill chunk) on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 500] [--config llama2_70b_gqa]
    python bench.py --config prefill_70b_gqa      (a prefill-chunk step, see prefill_bench)
    python bench.py --config swap_70b             (blocks out to pinned host memory and back, see swap_bench)
    python bench.py --config block_manager        (host bookkeeping of decode steps, see block_manager_bench)
    python bench.py --config cache_ops            (reshape_and_cache and copy_blocks per call, see cache_ops_bench)

A step is the whole hot path over one synthetic batch: copy-on-write block copies
(when the batch has any), the cache write of every sequence's new token, then
decode attention over the paged cache. All three run as one launch (pkv_decode_step
with cow_src); --cow-launch copies with copy_blocks first, and --separate times
copy_blocks, reshape_and_cache and paged_attention_decode as three launches. Inputs
are resident in HBM before timing.
Consecutive steps rotate over --replicas independent batches (own pools and block
tables), so each step reads KV bytes the previous steps did not touch: about 2 GB
lie between two reads of the same batch, far beyond the 256 MB last-level cache.

Prints one JSON line. `value` is KV-read GB/s of the whole step (algorithmic KV
bytes / step time); `roofline` reports the decode kernel alone, timed with HIP
events on the stream it runs on; `cpu_baseline` times the float64 CPU oracle on a
bounded sample of the same batch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X published HBM3E bandwidth
PEAK_MFMA_TFLOPS = 2500.0      # MI355X published dense bf16 / fp16 matrix-core rate
PEAK_HOST_LINK_GBS = 64.0      # PCIe 5.0 x16, one direction: the MI355X host link
CPU_SAMPLE_SECONDS = 12.0      # target length of the timed oracle sample
DECODE_SOURCES = ("paged_kv_cache_409_amd/csrc/decode_mfma.hip", "paged_kv_cache_409_amd/csrc/decode_valu.hip",
                  "paged_kv_cache_409_amd/csrc/decode_common.h", "paged_kv_cache_409_amd/csrc/pkv_device.h")


PREFILL_COMMON = ("paged_kv_cache_409_amd/csrc/prefill_common.h", "paged_kv_cache_409_amd/csrc/decode_common.h",
                  "paged_kv_cache_409_amd/csrc/pkv_device.h", "paged_kv_cache_409_amd/csrc/pkv_launch.h",
                  "paged_kv_cache_409_amd/build.py")


def prefill_kernel(kv_dtype: str):
    """(kernel name, sources) of the prefill kernel that serves a cache of this dtype."""
    if kv_dtype == "fp8_e4m3":
        return "paged_prefill_mfma", ("paged_kv_cache_409_amd/csrc/prefill_mfma.hip",) + PREFILL_COMMON
    return "paged_prefill_lds", ("paged_kv_cache_409_amd/csrc/prefill_lds.hip",) + PREFILL_COMMON


def kernel_source_hash(sources=DECODE_SOURCES) -> str:
    """Hash of a kernel's sources and of the compiler flags they are built with (common and per
    file; include paths, which differ between machines, left out): counters taken from any
    other build do not describe this one."""
    from paged_kv_cache_409_amd.build import COMMON, FILE_FLAGS, ROOT as BUILD_ROOT
    h = hashlib.sha256()
    h.update(" ".join(f for f in COMMON if not f.startswith(BUILD_ROOT)).encode())
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
        h.update(" ".join(FILE_FLAGS.get(os.path.basename(f), [])).encode())
    return h.hexdigest()[:16]


def load_traffic(config_name: str, kind: str = "decode", sources=DECODE_SOURCES):
    """HBM traffic of one launch from committed counter runs, if they match this kernel's sources."""
    path = os.path.join(ROOT, "profiles", f"{kind}_traffic_{config_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash(sources):
        return None
    return t.get("hbm_bytes_per_launch")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # A step is about 0.1 ms. The first few hundred steps of a run are slower than the
    # rest: after 10 warm-up steps the beam workload's timed steps ran about 10% slower,
    # after 50 about 3% (the 70B batch about 0.5%), after 400 no slower than later ones. 500
    # warm-up steps take about 55 ms, and 200 timed steps about 25 ms.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--config", default="llama2_70b_gqa")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seqs", type=int, default=0, help="sequences the oracle times (0: auto)")
    ap.add_argument("--separate", action="store_true",
                    help="write the new tokens with their own launch instead of inside the decode launch")
    ap.add_argument("--cow-launch", action="store_true",
                    help="copy the step's copy-on-write pairs with copy_blocks before the decode launch instead "
                         "of inside it")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain 1 GiB device-to-device copy instead (reference kernel for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: decode attention shards by kv head or sequence with no exchange, "
              "so one GPU's rate is the measure; use --gpus 1.", file=sys.stderr)
        return 2

    if args.config == "block_manager":
        return block_manager_bench(args)

    from workloads import BLOCK_SIZE_CONFIGS, CONFIGS, PREFILL_CONFIGS, SWAP_CONFIGS
    # The oracle's worker processes are forked now, before anything touches the GPU.
    pool = None
    if not (args.no_cpu_baseline or args.copy_calibration) and args.config not in SWAP_CONFIGS and \
            args.config != "cache_ops":
        pool = OraclePool()
    try:
        return gpu_bench(args, pool)
    finally:
        if pool is not None:
            pool.close()


def gpu_bench(args, pool) -> int:
    import torch

    import paged_kv_cache_409_amd as pkv
    from workloads import BLOCK_SIZE_CONFIGS, CONFIGS, PREFILL_CONFIGS, SHARD_CONFIGS, SWAP_CONFIGS, make_batch
    from workloads.gen import kv_bytes_logical, kv_bytes_unique

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        return copy_calibration(args, dev)
    if args.config in PREFILL_CONFIGS:
        return prefill_bench(args, PREFILL_CONFIGS[args.config], dev, pool)
    if args.config in SWAP_CONFIGS:
        return swap_bench(args, SWAP_CONFIGS[args.config], dev)
    if args.config == "cache_ops":
        return cache_ops_bench(args, dev)
    cfg = {**CONFIGS, **BLOCK_SIZE_CONFIGS, **SHARD_CONFIGS}[args.config]
    batches = [make_batch(cfg, dev, replica=r) for r in range(args.replicas)]
    lay = batches[0].layout
    # Replicas draw their own context lengths: each step counts the bytes of its own batch.
    # Algorithmic bytes are the distinct bytes a step must read (= logical unless blocks are shared).
    kv_alg_r = [kv_bytes_unique(cfg, b.layout) for b in batches]
    kv_log_r = [kv_bytes_logical(cfg, b.layout.context_lens) for b in batches]
    ws_bytes = pkv.workspace_size(cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                                  cfg.max_context_len, cfg.partition_size)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(b.q) for b in batches]
    n_pairs = len(lay.copy_pairs)

    # Copy-on-write: fused into the decode launch (cow_src) unless the step is timed in its
    # separate-launch forms (--separate, --cow-launch), where copy_blocks runs first.
    copy_launch = n_pairs > 0 and (args.separate or args.cow_launch)

    def decode(i):   # the step's decode launch (with its reduce launch when the context is split)
        b = batches[i % len(batches)]
        if args.separate:
            pkv.paged_attention_decode(outs[i % len(batches)], b.q, b.k_cache, b.v_cache, b.block_tables,
                                       b.context_lens, b.scale, cfg.max_context_len, b.k_scale, b.v_scale,
                                       cfg.partition_size, workspace=ws)
        else:
            pkv.decode_step(outs[i % len(batches)], b.q, b.k_cache, b.v_cache, b.new_k, b.new_v, b.slot_mapping,
                            b.block_tables, b.context_lens, b.scale, cfg.max_context_len, b.k_scale, b.v_scale,
                            cfg.partition_size, workspace=ws,
                            cow_src=None if (copy_launch or n_pairs == 0) else b.cow_src)

    def step(i, ev=None):
        b = batches[i % len(batches)]
        if copy_launch and len(b.copy_pairs):
            pkv.copy_blocks([b.k_cache], [b.v_cache], b.copy_pairs)
        if args.separate:
            pkv.reshape_and_cache(b.new_k, b.new_v, b.slot_mapping, b.k_cache, b.v_cache, b.k_scale, b.v_scale)
        if ev is not None:
            ev[0].record()
        decode(i)
        if ev is not None:
            ev[1].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Timed region: K whole steps back to back, bracketed by two events only.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record()
    for i in range(args.steps):
        step(args.warmup + i)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    step_bytes = sum(kv_alg_r[(args.warmup + i) % len(batches)] for i in range(args.steps)) / args.steps
    # Second pass: the decode launches of K steps alone, back to back, between two events on
    # their stream (the step's other launches stay out; repeating a batch's decode reads the
    # same bytes and writes the same new tokens).
    first = args.warmup + args.steps
    d_start = torch.cuda.Event(enable_timing=True)
    d_end = torch.cuda.Event(enable_timing=True)
    d_start.record()
    for i in range(args.steps):
        decode(first + i)
    d_end.record()
    torch.cuda.synchronize()
    dec_region_ms = d_start.elapsed_time(d_end)
    ev_bytes = sum(kv_alg_r[(first + i) % len(batches)] for i in range(args.steps))
    # Third pass: whole steps with each decode launch between its own pair of events (each pair
    # adds its own overhead, so these run a little longer).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        step(first + args.steps + i, evs[i])
    torch.cuda.synchronize()
    dec_ms = np.array([a.elapsed_time(b) for a, b in evs])
    dec_avg_ms = float(dec_ms.mean())
    # When a step is the decode launch alone, the back-to-back pass is that launch as the timed
    # region runs it. When a step has other launches too (copy-on-write pairs, or the separate
    # cache write), the decode inside the step is timed by its own events instead: run alone,
    # back to back, it can take a different time than it does inside the step.
    alone = not copy_launch and not args.separate
    timing = "back_to_back" if alone else "per_launch_events"
    ceiling = probe_ceiling(args, cfg, batches, kv_log_r, kv_alg_r, alone)
    ev_bytes_pairs = sum(kv_alg_r[(first + args.steps + i) % len(batches)] for i in range(args.steps))
    achieved = (ev_bytes / (dec_region_ms * 1e-3) if alone else ev_bytes_pairs / (float(dec_ms.sum()) * 1e-3)) / 1e9
    ceiling["frac_of_ceiling"] = round(achieved / ceiling["GBps"], 4)

    result = {
        "metric": "paged decode attention: achieved KV-read HBM GB/s (% of peak) and seqs/s",
        "value": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"q {cfg.dtype}, kv {cfg.kv_dtype}; fp32 accumulate",
        "data": "synthetic",
        "config": {
            "workload": cfg.description,
            "num_seqs": cfg.num_seqs, "num_q_heads": cfg.num_q_heads, "num_kv_heads": cfg.num_kv_heads,
            "head_dim": cfg.head_dim, "block_size": cfg.block_size, "max_context_len": cfg.max_context_len,
            "partition_tokens": pkv.partition_tokens(cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads,
                                                     cfg.max_context_len, cfg.partition_size),
            "kv_bytes_algorithmic_per_replica": kv_alg_r, "kv_bytes_logical_per_replica": kv_log_r,
            "copy_pairs": n_pairs,
            "replicas": args.replicas, "seed": cfg.seed, "parallelism": "single GPU",
            "step": "copy_blocks + reshape_and_cache + paged_attention_decode" if args.separate else
                    ("copy_blocks + decode_step (cache write fused into the decode launch)" if copy_launch else
                     "decode_step (cache write, and copy-on-write of the step's pairs via cow_src, fused into the "
                     "decode launch)"),
        },
        "seqs_per_s": round(cfg.num_seqs / (ms_per_step * 1e-3), 1),
        "decode_us": {"back_to_back": round(dec_region_ms / args.steps * 1e3, 2),
                      "mean": round(dec_avg_ms * 1e3, 2), "p10": round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
                      "p50": round(float(np.percentile(dec_ms, 50)) * 1e3, 2),
                      "p90": round(float(np.percentile(dec_ms, 90)) * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "timing": timing, "traffic": load_traffic(cfg.name),
                     "kernel": "paged_decode_mfma" if cfg.group_size > 1 else "paged_decode_valu",
                     "kernel_source_hash": kernel_source_hash(), "ceiling": ceiling},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(pool, cfg, batches[0], args.cpu_sample_seqs)
    print(json.dumps(result), flush=True)
    return 0


def unique_tile_tables(cfg, lay):
    """Block tables that name each distinct tile of a sharing group once: for every group
    of neighbouring sequences the matrix-core decode kernel puts in one workgroup, the
    distinct physical blocks of each logical block, in logical order (the tiles the decode
    reads once for all of their readers). Returns (block_tables, context_lens) with one
    row per group and a context of whole 16-token tiles."""
    P = cfg.block_size
    G = cfg.num_q_heads // cfg.num_kv_heads
    B = min(16 // G, 4) if G > 1 else 1
    rows = []
    for g0 in range(0, cfg.num_seqs, B):
        members = range(g0, min(g0 + B, cfg.num_seqs))
        nblk = [-(-int(lay.context_lens[s]) // P) for s in members]
        row = []
        for j in range(max(nblk)):
            seen = []
            for s, n in zip(members, nblk):
                if j < n and int(lay.block_tables[s, j]) not in seen:
                    seen.append(int(lay.block_tables[s, j]))
            row += seen
        rows.append(row)
    width = max(len(r) for r in rows)
    bt = np.zeros((len(rows), width), dtype=np.int32)
    for i, r in enumerate(rows):
        bt[i, :len(r)] = r
    ctx = np.array([len(r) * P for r in rows], dtype=np.int32)
    return bt, ctx


def probe_ceiling(args, cfg, batches, kv_log_r, kv_alg_r, back_to_back) -> dict:
    """Rate of the decode read pattern alone on this device: pkv_gather_probe reads the bytes a
    decode step over each replica reads (the same tiles through the same block tables, with
    the decode kernels' loads) and does no arithmetic. Timed like the decode launches: K
    launches back to back between two events, or each launch between its own pair.
    Where sequences share blocks, the probe reads each group's distinct tiles once (the
    decode reads shared blocks once per group), and the rate is counted in unique bytes."""
    import torch

    import paged_kv_cache_409_amd as pkv

    shared = any(a != l for a, l in zip(kv_alg_r, kv_log_r))
    inputs = []
    for b in batches:
        if shared:
            bt, ctx = unique_tile_tables(cfg, b.layout)
            dev = b.k_cache.device
            inputs.append((torch.from_numpy(bt).to(dev), torch.from_numpy(ctx).to(dev), int(ctx.max())))
        else:
            inputs.append((b.block_tables, b.context_lens, cfg.max_context_len))
    sinks = [torch.zeros((c.shape[0], cfg.num_kv_heads), dtype=torch.int32, device=b.k_cache.device)
             for b, (_, c, _) in zip(batches, inputs)]

    def run(i):
        b = batches[i % len(batches)]
        bt, ctx, mx = inputs[i % len(batches)]
        pkv.gather_probe(b.k_cache, b.v_cache, bt, ctx, mx, sinks[i % len(batches)])

    for i in range(min(args.warmup, 4)):
        run(i)
    if back_to_back:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            run(i)
        e1.record()
        torch.cuda.synchronize()
        ms = np.full(args.steps, e0.elapsed_time(e1) / args.steps)
    else:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for i in range(args.steps):
            evs[i][0].record()
            run(i)
            evs[i][1].record()
        torch.cuda.synchronize()
        ms = np.array([a.elapsed_time(b) for a, b in evs])
    counted = kv_alg_r if shared else kv_log_r
    read = sum(counted[i % len(batches)] for i in range(args.steps))
    what = ("the distinct K/V tiles of each group of neighbouring sequences (what the decode reads once for all "
            "readers) through the decode kernels' loads and no arithmetic (unique bytes; pkv_gather_probe)") if shared \
        else ("the K/V tiles of every context read through the block tables with the decode kernels' "
              "loads and no arithmetic (logical bytes; pkv_gather_probe)")
    return {"kernel": "gather_probe", "GBps": round(read / (float(ms.sum()) * 1e-3) / 1e9, 1), "what": what,
            "us": round(float(ms.mean()) * 1e3, 2), "timing": "back_to_back" if back_to_back else "per_launch_events"}


def prefill_flops(cfg, lay) -> float:
    """Algorithmic matrix flops of a prefill chunk: new token i of sequence s attends to
    ctx_s - n_s + i + 1 keys, each costing 2 D flops for its score and 2 D for its
    share of the output, per query head."""
    n = np.diff(lay.query_start_loc).astype(np.int64)
    prefix = lay.context_lens.astype(np.int64) - n
    keys = int((n * prefix + n * (n + 1) // 2).sum())
    return 4.0 * cfg.head_dim * cfg.num_q_heads * keys


def prefill_bench(args, cfg, dev, pool) -> int:
    """One prefill-chunk step: the cache write of every sequence's chunk of new tokens,
    then causal attention of the chunk over the paged cache. `value` is matrix TFLOP/s of
    the whole step (algorithmic flops / step time); `roofline` reports the attention
    kernel alone against the dense bf16/fp16 matrix-core peak."""
    import torch

    import paged_kv_cache_409_amd as pkv
    from workloads import make_batch

    batches = [make_batch(cfg, dev, replica=r) for r in range(args.replicas)]
    lay = batches[0].layout
    # Replicas draw their own context lengths, so each has its own flop count.
    flops_r = [prefill_flops(cfg, b.layout) for b in batches]
    T = int(lay.query_start_loc[-1])
    max_q = [int(np.diff(b.layout.query_start_loc).max()) for b in batches]
    outs = [torch.empty_like(b.q) for b in batches]

    def attention(i):
        b = batches[i % len(batches)]
        pkv.paged_attention_prefill(outs[i % len(batches)], b.q, b.k_cache, b.v_cache, b.block_tables,
                                    b.context_lens, b.query_start_loc, b.scale, max_q[i % len(batches)],
                                    b.k_scale, b.v_scale)

    def step(i, ev=None):
        b = batches[i % len(batches)]
        pkv.reshape_and_cache(b.new_k, b.new_v, b.slot_mapping, b.k_cache, b.v_cache, b.k_scale, b.v_scale)
        if ev is not None:
            ev[0].record()
        attention(i)
        if ev is not None:
            ev[1].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record()
    for i in range(args.steps):
        step(args.warmup + i)
    t_end.record()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    step_flops = sum(flops_r[(args.warmup + i) % len(batches)] for i in range(args.steps)) / args.steps
    # Roofline: the attention launches of K steps alone, back to back, between two events.
    first = args.warmup + args.steps
    a_start = torch.cuda.Event(enable_timing=True)
    a_end = torch.cuda.Event(enable_timing=True)
    a_start.record()
    for i in range(args.steps):
        attention(first + i)
    a_end.record()
    torch.cuda.synchronize()
    pf_region_ms = a_start.elapsed_time(a_end)
    b2b_flops = sum(flops_r[(first + i) % len(batches)] for i in range(args.steps))
    # Whole steps with each attention launch between its own pair of events (reported beside
    # the roofline). Each pair adds a few µs of its own: in kernel traces the attention takes
    # the same time back to back as inside whole steps after the chunk's cache write, and the
    # pairs read longer than both.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        step(first + args.steps + i, evs[i])
    torch.cuda.synchronize()
    pf_ms = np.array([a.elapsed_time(b) for a, b in evs])
    pf_avg_ms = float(pf_ms.mean())
    achieved = b2b_flops / (pf_region_ms * 1e-3) / 1e12
    kernel, sources = prefill_kernel(cfg.kv_dtype)
    result = {
        "metric": "paged prefill-chunk attention: achieved matrix TFLOP/s (% of dense bf16 peak) and tokens/s",
        "value": round(step_flops / (ms_per_step * 1e-3) / 1e12, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"q {cfg.dtype}, kv {cfg.kv_dtype}; fp32 accumulate",
        "data": "synthetic",
        "config": {
            "workload": cfg.description,
            "num_seqs": cfg.num_seqs, "num_q_heads": cfg.num_q_heads, "num_kv_heads": cfg.num_kv_heads,
            "head_dim": cfg.head_dim, "block_size": cfg.block_size, "new_tokens": T, "max_query_len": max(max_q),
            "context_lens_replica0": lay.context_lens.tolist(),
            "flops_algorithmic_per_replica": flops_r, "flops_algorithmic_mean": round(step_flops),
            "replicas": args.replicas, "seed": cfg.seed, "parallelism": "single GPU",
            "step": "reshape_and_cache (chunk) + paged_attention_prefill",
        },
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "prefill_us": {"back_to_back": round(pf_region_ms / args.steps * 1e3, 2), "mean": round(pf_avg_ms * 1e3, 2), "p10": round(float(np.percentile(pf_ms, 10)) * 1e3, 2),
                       "p50": round(float(np.percentile(pf_ms, 50)) * 1e3, 2),
                       "p90": round(float(np.percentile(pf_ms, 90)) * 1e3, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_MFMA_TFLOPS, 4), "timing": "back_to_back",
                     "traffic": load_traffic(cfg.name, "prefill", sources),
                     "kernel": kernel, "kernel_source_hash": kernel_source_hash(sources)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = prefill_cpu_baseline(pool, cfg, batches[0])
    print(json.dumps(result), flush=True)
    return 0


def prefill_cpu_baseline(pool, cfg, b):
    """Time the float64 prefill oracle over the whole batch, one (sequence, kv head) per task
    on the worker processes."""
    ctx, qsl = b.context_lens.cpu().numpy(), b.query_start_loc.cpu().numpy()
    n = np.diff(qsl).astype(np.int64)
    work = n * (ctx - n) + n * (n + 1) // 2
    G = cfg.num_q_heads // cfg.num_kv_heads
    # the GPU wrote the chunk into the pool during timing
    arrays = dict(q=host_bits(b.q), kc=host_bits(b.k_cache), vc=host_bits(b.v_cache),
                  bt=b.block_tables.cpu().numpy(), ctx=ctx, qsl=qsl)
    meta = dict(scale=cfg.scale, dtype=cfg.dtype, kv_dtype=cfg.kv_dtype, k_scale=b.k_scale, v_scale=b.v_scale,
                group=G)
    tasks = [(int(s), g) for s in np.argsort(-work) for g in range(cfg.num_kv_heads)]      # longest first
    dt, passes = pool.timed_passes(arrays, meta, "prefill", tasks)
    flops = 4.0 * cfg.head_dim * cfg.num_q_heads * float(work.sum())
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "tokens_per_s": round(float(n.sum()) / dt, 2),
            "cores": pool.workers, "cpus_visible": pool.visible, "cpu_model": pool.model, "kind": "oracle",
            "sample": f"all {cfg.num_seqs} sequences (all rows and heads), float64 numpy oracle, one (sequence, "
                      f"kv head) per task on {pool.workers} worker processes; {passes} timed pass(es), "
                      f"median round {dt:.3f} s per pass"}


def cache_ops_bench(args, dev) -> int:
    """The two cache operations of the step on their own, per call: reshape_and_cache of a
    70B decode step's 256 new tokens (bf16), of the 70B prefill batch's 4096 chunk tokens,
    and of the beam step's 256 tokens into an fp8 cache (with the encode); copy_blocks of the
    beam step's copy-on-write pairs. Each case rotates over --replicas batches. `us` is the
    time per call of K calls back to back (one event pair around all of them); `us_event` the
    mean of per-call event pairs, which adds the launch's dispatch latency. Bytes are what the
    call must move: rows read and slots written (plus the slot list), or source blocks read
    and destination blocks written."""
    import torch

    import paged_kv_cache_409_amd as pkv
    from workloads import CONFIGS, PREFILL_CONFIGS, make_batch

    def timed(call, n_rep):
        for i in range(args.warmup):
            call(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(args.steps):
            call(i)
        b.record()
        torch.cuda.synchronize()
        per_call = a.elapsed_time(b) / args.steps
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for i in range(args.steps):
            evs[i][0].record()
            call(i)
            evs[i][1].record()
        torch.cuda.synchronize()
        ev = np.array([x.elapsed_time(y) for x, y in evs])
        return per_call, float(ev.mean()), float(np.percentile(ev, 50))

    cases = []

    def add(name, workload, nbytes, call):
        ms, ev_mean, ev_p50 = timed(call, args.steps)
        gbs = nbytes / (ms * 1e-3) / 1e9
        cases.append({"op": name, "workload": workload, "bytes_per_call": int(nbytes), "us": round(ms * 1e3, 2),
                      "us_event": {"mean": round(ev_mean * 1e3, 2), "p50": round(ev_p50 * 1e3, 2)},
                      "GBps": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)})

    def write_case(cfg, workload):
        bs = [make_batch(cfg, dev, replica=r) for r in range(args.replicas)]
        T, Hkv, D = bs[0].new_k.shape
        kv_b = 1 if cfg.kv_dtype == "fp8_e4m3" else 2
        nbytes = T * Hkv * D * (2 * 2 + 2 * kv_b) + T * 8

        def call(i):
            b = bs[i % len(bs)]
            pkv.reshape_and_cache(b.new_k, b.new_v, b.slot_mapping, b.k_cache, b.v_cache, b.k_scale, b.v_scale)
        add("reshape_and_cache", workload, nbytes, call)
        return bs

    write_case(CONFIGS["llama2_70b_gqa"], "Llama-2-70B GQA decode step: 256 new tokens x 8 kv heads x D 128, bf16")
    write_case(PREFILL_CONFIGS["prefill_70b_gqa"],
               "Llama-2-70B GQA prefill chunks: 8 x 512 = 4096 new tokens x 8 kv heads x D 128, bf16")
    beams = write_case(CONFIGS["beam_cow"], "beam CoW decode step: 256 new tokens x 8 kv heads x D 128, "
                                            "bf16 in, fp8 E4M3 cache (IEEE division by the scale, RNE)")
    n_pairs = len(beams[0].copy_pairs)
    block_bytes = beams[0].k_cache[0].numel() * beams[0].k_cache.element_size()

    def copy_call(i):
        b = beams[i % len(beams)]
        pkv.copy_blocks([b.k_cache], [b.v_cache], b.copy_pairs)
    add("copy_blocks", f"beam CoW decode step: {n_pairs} copy-on-write pairs, one layer, K and V, "
                       f"{block_bytes} bytes per block per tensor (fp8)", 2 * 2 * n_pairs * block_bytes, copy_call)

    result = {
        "metric": "cache write and copy-on-write: us per call and GB/s",
        "value": cases[0]["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(cases[0]["us"] / 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 rows; bf16 or fp8 E4M3 caches", "data": "synthetic",
        "config": {"workload": "reshape_and_cache and copy_blocks at the decode, prefill and beam workloads' sizes "
                               "(value: the 70B decode step's cache write)",
                   "replicas": args.replicas, "parallelism": "single GPU"},
        "cases": cases,
        "roofline": {"bound": "hbm", "achieved": cases[0]["GBps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": cases[0]["frac_of_hbm_peak"], "traffic": None, "kernel": "reshape_and_cache_kernel",
                     "note": "launch-bound at these sizes: a few MB per call"},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cache_write_cpu_baseline(CONFIGS["beam_cow"], beams[0])
    print(json.dumps(result), flush=True)
    return 0


def cache_write_cpu_baseline(cfg, b):
    """The reshape_and_cache oracle on the beam step's 256 tokens (fp8 encode), one thread.
    The oracle returns new pools, so each call also copies the two pools."""
    from oracle import cache_ops
    _, visible, model = host_cpu()
    k, v, kc, vc = host_bits(b.new_k), host_bits(b.new_v), host_bits(b.k_cache), host_bits(b.v_cache)
    sm = b.slot_mapping.cpu().numpy()
    run = lambda: cache_ops.reshape_and_cache(k, v, sm, kc, vc, cfg.dtype, cfg.kv_dtype, b.k_scale, b.v_scale)
    run()
    times = []
    while len(times) < 3 and sum(times) <= CPU_SAMPLE_SECONDS:
        t0 = time.perf_counter()
        run()
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    T, Hkv, D = k.shape
    nbytes = T * Hkv * D * (2 * 2 + 2 * 1) + T * 8
    return {"value": round(nbytes / dt / 1e9, 6), "unit": "GB/s", "us_per_call": round(dt * 1e6, 1), "cores": 1,
            "cpus_visible": visible, "cpu_model": model, "kind": "oracle",
            "sample": f"reshape_and_cache of the beam step's {T} tokens into fp8 pools (the oracle copies both "
                      f"{kc.nbytes} byte pools per call), numpy on one host thread; median of {len(times)} runs"}


def swap_bench(args, cfg, dev) -> int:
    """One swap step: a preempted request's blocks (scattered, every layer, K and V) go out
    to pinned host memory, then come back into other free GPU blocks. `value` is bytes moved
    over the host link per second, both directions together; `roofline` compares it with
    the link's one-direction peak (the two directions run one after the other). Beside it,
    one contiguous runtime copy of the same size each way gives the link rate the DMA
    engines reach."""
    import torch

    import paged_kv_cache_409_amd as pkv
    from workloads import make_swap_pairs, make_swap_pools

    gpu = make_swap_pools(cfg, "gpu", dev)
    host = make_swap_pools(cfg, "host", dev, pin=True)
    gk, gv = [k for k, _ in gpu], [v for _, v in gpu]
    hk, hv = [k for k, _ in host], [v for _, v in host]
    out_np, in_np = make_swap_pairs(cfg)
    out_pairs, in_pairs = torch.from_numpy(out_np).to(dev), torch.from_numpy(in_np).to(dev)
    nbytes = cfg.bytes_per_direction

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        pkv.swap_blocks(gk, gv, hk, hv, out_pairs)
        if ev is not None:
            ev[1].record()
        pkv.swap_blocks(hk, hv, gk, gv, in_pairs)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    out_ms = np.array([a.elapsed_time(b) for a, b, _ in evs])
    in_ms = np.array([b.elapsed_time(c) for _, b, c in evs])
    # Contiguous runtime copies of the same size, for the DMA engines' link rate.
    dsrc = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    hbuf = torch.empty(nbytes, dtype=torch.uint8).pin_memory()
    hbuf.copy_(dsrc, non_blocking=True)
    torch.cuda.synchronize()
    c0, c1, c2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    c0.record()
    hbuf.copy_(dsrc, non_blocking=True)
    c1.record()
    dsrc.copy_(hbuf, non_blocking=True)
    c2.record()
    torch.cuda.synchronize()
    dma_out, dma_in = c0.elapsed_time(c1), c1.elapsed_time(c2)
    gbs = lambda ms: round(nbytes / (ms * 1e-3) / 1e9, 2)
    achieved = 2 * nbytes / ((out_ms.mean() + in_ms.mean()) * 1e-3) / 1e9
    result = {
        "metric": "block swap GPU <-> pinned host: achieved GB/s over the host link (% of its one-direction peak)",
        "value": round(2 * nbytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"kv {cfg.kv_dtype} (bytes moved as they are)",
        "data": "synthetic",
        "config": {"workload": cfg.description, "num_layers": cfg.num_layers, "num_kv_heads": cfg.num_kv_heads,
                   "head_dim": cfg.head_dim, "block_bytes": cfg.block_bytes, "blocks_per_layer": cfg.swap_blocks,
                   "bytes_per_direction": nbytes, "parallelism": "single GPU",
                   "step": "swap_blocks GPU->host (out) + swap_blocks host->GPU (in)"},
        "swap_out_GBps": gbs(float(out_ms.mean())), "swap_in_GBps": gbs(float(in_ms.mean())),
        "swap_us": {"out_mean": round(float(out_ms.mean()) * 1e3, 1), "in_mean": round(float(in_ms.mean()) * 1e3, 1)},
        "dma_contiguous_GBps": {"out": gbs(dma_out), "in": gbs(dma_in)},
        "roofline": {"bound": "host-link", "achieved": round(achieved, 2), "peak": PEAK_HOST_LINK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HOST_LINK_GBS, 4), "traffic": None,
                     "kernel": "move_blocks_kernel"},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = swap_cpu_baseline(cfg, gk, gv, hk, hv, out_np)
    print(json.dumps(result), flush=True)
    return 0


def swap_cpu_baseline(cfg, gk, gv, hk, hv, out_pairs):
    """Time the swap oracle on host copies of the pools. The oracle copies the destination
    pools and then every pair's blocks in one sequential pass, so it runs on one thread:
    median of three whole swap-outs after one warm-up (one timed run when a run is longer
    than CPU_SAMPLE_SECONDS)."""
    import torch

    from oracle import cache_ops
    to_np = lambda ts: [t.detach().cpu().numpy() if t.element_size() == 1 else
                        t.detach().cpu().view(torch.int16).numpy() for t in ts]
    sk, sv, dk, dv = to_np(gk), to_np(gv), to_np(hk), to_np(hv)
    _, visible, model = host_cpu()
    cache_ops.swap_blocks(sk, sv, dk, dv, out_pairs)          # warm-up
    times = []
    while len(times) < 3 and sum(times) <= CPU_SAMPLE_SECONDS:
        t0 = time.perf_counter()
        cache_ops.swap_blocks(sk, sv, dk, dv, out_pairs)
        times.append(time.perf_counter() - t0)
    dt, passes = float(np.median(times)), len(times)
    return {"value": round(cfg.bytes_per_direction / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
            "cpus_visible": visible, "cpu_model": model, "kind": "oracle",
            "sample": f"one swap-out of the whole case ({cfg.bytes_per_direction} bytes) between host arrays, "
                      f"numpy oracle on one host thread (it is one sequential pass); median of {passes} run(s), "
                      f"{dt:.2f} s each"}


def block_manager_bench(args) -> int:
    """Host bookkeeping of decode steps with the C++ block manager: 64 requests whose
    500-token prompts share a 256-token system prompt (prefix caching on), 4 beams each;
    a step appends one token to each of the 256 beams (slots, copy-on-write pairs) and
    builds their block tables. Timed against the Python block pool the workloads are laid
    out with, on the same history. No GPU is involved."""
    from paged_kv_cache_409_amd.block_manager import BlockManager
    from workloads.blocks import BlockPool, Sequence

    R, B, prompt_len, sys_len, P, NB = 64, 4, 500, 256, 16, 32768
    steps = max(args.steps, 1) * 4
    rng = np.random.default_rng(40910)
    system = rng.integers(0, 32000, size=sys_len).astype(np.int32)
    prompts = [np.concatenate([system, rng.integers(0, 32000, size=prompt_len - sys_len).astype(np.int32)])
               for _ in range(R)]
    max_blocks = (prompt_len + steps + P - 1) // P

    def run_cpp():
        bm = BlockManager(NB, block_size=P, prefix_caching=True)
        cached = 0
        for r in range(R):
            _, c = bm.add_sequence(1000 * r, prompt_len, prompts[r])
            cached += c
            for b in range(B):
                bm.fork(1000 * r, 1000 * r + 1 + b)
            bm.free(1000 * r)
        ids = np.array([1000 * r + 1 + b for r in range(R) for b in range(B)], dtype=np.int64)
        tok = np.zeros(len(ids), dtype=np.int32)
        t0 = time.perf_counter()
        copies = 0
        for _ in range(steps):
            _, pairs = bm.append_batch(ids, tok)
            copies += len(pairs)
            bm.block_tables(ids, max_blocks)
        return time.perf_counter() - t0, copies, cached

    def run_python():
        pool = BlockPool(NB, P)
        seqs = []
        for r in range(R):
            root = Sequence(pool)
            root.extend(prompt_len)
            seqs += [root.fork() for _ in range(B)]
            root.free()
        t0 = time.perf_counter()
        for _ in range(steps):
            for sq in seqs:
                sq.append_slot()
            tables = np.zeros((len(seqs), max_blocks), dtype=np.int32)
            for i, sq in enumerate(seqs):
                tables[i, :len(sq.blocks)] = sq.blocks
        return time.perf_counter() - t0

    dt, copies, cached = run_cpp()
    dt_py = run_python()
    n = R * B * steps
    result = {
        "metric": "block-manager bookkeeping of decode steps: sequence-steps/s (host, C++)",
        "value": round(n / dt, 1), "unit": "sequence-steps/s", "n_gpus": 0, "steps": steps, "warmup": 0,
        "ms_per_step": round(dt / steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32 / int64 (block ids, slots)", "data": "synthetic",
        "config": {"workload": f"{R} requests x {B} beams, {prompt_len}-token prompts sharing a {sys_len}-token "
                               f"system prompt, prefix caching on, {NB}-block pool, block size {P}",
                   "copy_on_write_pairs": copies, "prompt_tokens_served_from_cache": cached,
                   "step": "append one token to every beam (slots, copy pairs) + block tables of all beams"},
        "us_per_step": round(dt / steps * 1e6, 1),
        "roofline": None,
        "cpu_baseline": {"value": round(n / dt_py, 1), "unit": "sequence-steps/s", "cores": 1,
                         "kind": "python reference pool (workloads/blocks.py)",
                         "sample": f"the same {steps} steps without prefix caching, {dt_py:.2f} s"},
    }
    print(json.dumps(result), flush=True)
    return 0


def copy_calibration(args, dev) -> int:
    """A plain 1 GiB copy of known size: its HBM counters calibrate the decode kernel's, and its
    rate is the measured copy ceiling of this GPU."""
    import torch
    nbytes = 1 << 30
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(args.steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "ms_per_copy": round(ms, 4),
                      "read_plus_write_GBps": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}), flush=True)
    return 0


def host_cpu():
    """(workers, CPUs visible to this process, CPU model) for the oracle baselines. The
    workers are the CPUs this process may run on, capped by OMP_NUM_THREADS where the machine
    sets it (the host share of one GPU)."""
    visible = len(os.sched_getaffinity(0))
    cap = int(os.environ.get("OMP_NUM_THREADS") or visible)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return max(1, min(visible, cap)), visible, model


_ORACLE_INPUTS = {}


def _oracle_worker_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)       # one BLAS thread per worker process


def _oracle_task(task):
    """One oracle task in a worker process: the inputs are memory-mapped .npy files in
    task[0] (loaded once per process), task[1] names the oracle, task[2:] its work item."""
    import numpy as np

    from oracle import attention
    folder, kind = task[0], task[1]
    if folder not in _ORACLE_INPUTS:
        _ORACLE_INPUTS.clear()
        _ORACLE_INPUTS[folder] = {f[:-4]: np.load(os.path.join(folder, f), mmap_mode="r")
                                  for f in os.listdir(folder) if f.endswith(".npy")}
    a = _ORACLE_INPUTS[folder]
    meta = json.load(open(os.path.join(folder, "meta.json")))
    if kind == "decode":
        attention.paged_decode_attention(a["q"], a["kc"], a["vc"], a["bt"], a["ctx"], meta["scale"], meta["dtype"],
                                         meta["kv_dtype"], meta["k_scale"], meta["v_scale"], seqs=[task[2]])
    else:                              # one kv head of one prefill sequence
        s, g, G = task[2], task[3], meta["group"]
        attention.paged_prefill_attention(a["q"][:, g * G:(g + 1) * G], a["kc"][:, g:g + 1], a["vc"][:, g:g + 1],
                                          a["bt"], a["ctx"], a["qsl"], meta["scale"], meta["dtype"],
                                          meta["kv_dtype"], meta["k_scale"], meta["v_scale"], seqs=[s])
    return 0


class OraclePool:
    """Worker processes for the CPU baseline. They are forked before this process touches
    the GPU (a process that has initialised the GPU must not be forked or exec'd) and
    never use it; the inputs reach them as .npy files they memory-map."""

    def __init__(self):
        import multiprocessing
        self.workers, self.visible, self.model = host_cpu()
        self.pool = multiprocessing.get_context("fork").Pool(self.workers, initializer=_oracle_worker_init)

    def timed_passes(self, arrays: dict, meta: dict, kind: str, items):
        """Wall time of one whole pass over `items`: after a warm-up over the first items, the
        median of three timed rounds, each as many whole passes as take about a third of
        CPU_SAMPLE_SECONDS of the workers' time together (so that the sample is about
        CPU_SAMPLE_SECONDS of CPU work); one single pass when a pass is longer than that.
        Returns (seconds per pass, passes timed)."""
        import shutil
        import tempfile
        need = sum(int(a.nbytes) for a in arrays.values())
        # memory-backed files where there is room for them twice over, else the temporary folder
        shm = "/dev/shm" if os.path.isdir("/dev/shm") and shutil.disk_usage("/dev/shm").free > 2 * need else None
        folder = tempfile.mkdtemp(prefix="pkv_oracle_", dir=shm)
        try:
            for name, arr in arrays.items():
                np.save(os.path.join(folder, name + ".npy"), np.ascontiguousarray(arr))
            with open(os.path.join(folder, "meta.json"), "w") as f:
                json.dump(meta, f)
            tasks = [(folder, kind, *it) for it in items]

            def one_pass(ts):
                t0 = time.perf_counter()
                self.pool.map(_oracle_task, ts, chunksize=1)
                return time.perf_counter() - t0

            one_pass(tasks[:self.workers] * 2)
            first = one_pass(tasks)
            if first * self.workers > CPU_SAMPLE_SECONDS:
                return first, 1
            reps = max(1, int(CPU_SAMPLE_SECONDS / 3 / (first * self.workers)))
            rounds = [one_pass(tasks * reps) / reps for _ in range(3)]
            return float(np.median(rounds)), 3 * reps
        finally:
            shutil.rmtree(folder, ignore_errors=True)

    def close(self):
        self.pool.terminate()
        self.pool.join()


def host_bits(t):
    """Raw storage bits of a tensor as a host numpy array (uint16 for 16-bit types)."""
    import torch
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if t.element_size() == 2 else t.view(torch.uint8).numpy()


def cpu_baseline(pool, cfg, b, sample_seqs: int):
    """Time the float64 oracle over the whole batch (or its first `sample_seqs` sequences),
    one sequence per task on the worker processes."""
    # The pool already holds this step's copies and new tokens (the GPU wrote them during timing).
    ctx = b.context_lens.cpu().numpy()
    arrays = dict(q=host_bits(b.q), kc=host_bits(b.k_cache), vc=host_bits(b.v_cache),
                  bt=b.block_tables.cpu().numpy(), ctx=ctx)
    meta = dict(scale=cfg.scale, dtype=cfg.dtype, kv_dtype=cfg.kv_dtype, k_scale=b.k_scale, v_scale=b.v_scale)
    seqs = list(range(sample_seqs if 0 < sample_seqs < cfg.num_seqs else cfg.num_seqs))
    dt, passes = pool.timed_passes(arrays, meta, "decode", [(s,) for s in seqs])
    kv = int(ctx[seqs].astype(np.int64).sum()) * 2 * cfg.num_kv_heads * cfg.head_dim * (
        1 if cfg.kv_dtype == "fp8_e4m3" else 2)
    what = f"all {cfg.num_seqs} sequences" if len(seqs) == cfg.num_seqs else f"{len(seqs)} of {cfg.num_seqs} sequences"
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "seqs_per_s": round(len(seqs) / dt, 2),
            "cores": pool.workers, "cpus_visible": pool.visible, "cpu_model": pool.model, "kind": "oracle",
            "sample": f"{what} (all heads, logical KV bytes), float64 numpy oracle, one sequence per task on "
                      f"{pool.workers} worker processes; {passes} timed pass(es), median round {dt:.3f} s per pass"}


if __name__ == "__main__":
    sys.exit(main())
