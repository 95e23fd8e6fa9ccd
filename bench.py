#!/usr/bin/env python3
"""Throughput of the paged decode path on one MI355X.

Workload: the Llama-7B-shaped single-layer decode batch (96 sequences, 32 heads x
128, block size 16, contexts uniform in [300, 2048], fp16 KV and q, fp32
accumulation, blocks scattered at random over a pool of 110% of the blocks needed).

One step = one pass of the hot path over that batch: each sequence's newest K/V row
appended at its position and the decode over the contexts that count it, in one
launch (pa_decode_append: the 96 rows stored by workgroups of their own while the
attention folds them from registers; bit-identical to pa_cache_append followed by
pa_decode, which is timed beside it).  The batch has no shared blocks, so no block
copy is due.

Printed: one JSON line.  value = decode KV bytes per step / time per step (GB/s),
with every input resident in HBM.  roofline: that launch (the step's one kernel,
the decode partition pass with the append fused) timed with HIP events on the
stream it runs on; achieved = its algorithmic bytes (live K and V rows, plus the
appended rows read and written) / its average duration, against 8 TB/s.
cpu_baseline: the CPU oracle on a bounded sample of the same batch.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "pa_decode KV GB/s & % of MI355X HBM peak; decode seq-steps/s (1 GPU)"

# HBM bytes per launch of the step's kernel on this workload (seed 2: the partition
# pass with the 96 rows' append fused, pa_decode_append), from two
# rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE) scaled by the same counters of a
# known-size block copy (FETCH_SIZE x 1.9987, WRITE_SIZE x 1.0000); the commands and
# raw values are in profiles/decode_partitions_llama7b_pmc.md.  Valid only for the
# kernel sources and launch policy they were taken on (sha256 of the kernel file, the
# launch header whose constants the kernels use, and the host code that picks the
# partition length and the workgroup size of a launch).
MEASURED_TRAFFIC = {
    "kernel_source_sha256": "2b83b8b5b54a40f2c693b921b9f74f62f420c66ebc8555da26f110e0610434b8",
    "seed": 2,
    "partition_tokens": 2048,
    "read_bytes": 1926994397,
    "write_bytes": 2359259,
}
KERNEL_SOURCES = [os.path.join(os.path.dirname(os.path.abspath(__file__)),
                               "paged_kv_cache_414_amd", "csrc", name)
                  for name in ("pa_kernels.hip", "pa_launch.h", "pa_api.cpp")]


def kernel_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(seed, partition_tokens):
    """Counter-measured HBM bytes per launch, or None if the kernel sources or the
    workload differ from the ones the counters were taken on."""
    sha = kernel_sources_sha256()
    t = MEASURED_TRAFFIC
    if sha != t["kernel_source_sha256"] or seed != t["seed"] or partition_tokens != t["partition_tokens"]:
        return None
    return t["read_bytes"] + t["write_bytes"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--partition", type=int, default=0, help="tokens per partition, 0 = auto")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of each leg of the CPU-oracle sample (0 = skip)")
    ap.add_argument("--no-mixes", dest="mixes", action="store_false",
                    help="skip the continuous-batching and shared-prefix step mixes")
    ap.add_argument("--no-extras", dest="extras", action="store_false",
                    help="skip the long-context, shared-prefix, fp32, graph and swap sections")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="skip the graph-replay section only")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one pa_block_copy of a known size (counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the benchmark: pa_decode by block size and head dim")
    ap.add_argument("--graph-only", action="store_true",
                    help="instead of the benchmark: the graph-replayed vs eager small-batch steps")
    ap.add_argument("--quiet", action="store_true")
    return ap.parse_args()


def log(args, msg):
    if not args.quiet:
        print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_launches(fn, n, torch):
    """Average ms of ``fn`` over n back-to-back launches, HIP events on the current
    stream (the stream every entry point here launches on)."""
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(n):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / n


def launch_spread(fn, n, torch):
    """Per-launch ms of ``fn`` over n back-to-back launches, an event pair around each
    on the current stream: 10th percentile, median and 90th percentile."""
    stream = torch.cuda.current_stream()
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n)]
    torch.cuda.synchronize()
    for a, b in pairs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in pairs])
    p10, p50, p90 = np.percentile(t, [10, 50, 90])
    return {"launches": n, "p10_ms": round(float(p10), 5), "median_ms": round(float(p50), 5),
            "p90_ms": round(float(p90), 5)}


# Worker processes the multi-core leg of the CPU baseline may use at most: the host cores
# a one-GPU node of an MI355X machine provides (16), whatever more the affinity mask shows.
CPU_POOL_LIMIT = 16


def _oracle_pairs(batch, budget_s, worker, workers, start):
    """(pairs, tokens) the oracle finished between `start` and `start + budget_s`
    (time.time() clock), taking the batch's (seq, head) pairs worker, worker +
    workers, ... in order and repeating the batch."""
    import oracle

    h_count = batch.num_heads
    n_pairs = batch.num_seqs * h_count
    pairs = tokens = 0
    i = worker
    while time.time() < start + budget_s:
        s, h = divmod(i % n_pairs, h_count)
        oracle.decode_one(batch.q[s, h], batch.k_pool, batch.v_pool, batch.block_tables[s],
                          batch.context_lens[s], h, batch.scale)
        tokens += int(batch.context_lens[s])
        pairs += 1
        i += workers
    return pairs, tokens


class _MappedBatch:
    """The arrays of a decode batch the oracle reads, memory-mapped read-only from the
    files a parent process wrote (no copy per worker)."""

    def __init__(self, folder, meta):
        for name in ("q", "k_pool", "v_pool", "block_tables", "context_lens"):
            setattr(self, name, np.load(os.path.join(folder, name + ".npy"), mmap_mode="r"))
        self.num_seqs, self.num_heads, self.scale = meta


def _pool_worker(folder, meta, budget_s, worker, workers, start):
    """One worker process of the multi-core leg (a fresh interpreter)."""
    from threadpoolctl import threadpool_limits

    batch = _MappedBatch(folder, meta)
    with threadpool_limits(limits=1):
        while time.time() < start:
            time.sleep(0.01)
        return _oracle_pairs(batch, budget_s, worker, workers, start)


def _multi_core_leg(batch, budget_s, workers):
    """The oracle over the batch's pairs in `workers` fresh worker processes (spawned,
    so none of them inherits this process's GPU state), all starting at one wall-clock
    time and stopping `budget_s` seconds later; (pairs, tokens) summed."""
    import multiprocessing
    import shutil
    import tempfile
    from concurrent.futures import ProcessPoolExecutor

    folder = tempfile.mkdtemp(prefix="pa_oracle_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    try:
        for name in ("q", "k_pool", "v_pool", "block_tables", "context_lens"):
            np.save(os.path.join(folder, name + ".npy"), np.ascontiguousarray(getattr(batch, name)))
        meta = (batch.num_seqs, batch.num_heads, batch.scale)
        ctx = multiprocessing.get_context("spawn")
        with ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as pool:
            start = time.time() + 5.0  # time for every worker to start and map the files
            futs = [pool.submit(_pool_worker, folder, meta, budget_s, w, workers, start)
                    for w in range(workers)]
            done = [f.result() for f in futs]
    finally:
        shutil.rmtree(folder, ignore_errors=True)
    return sum(p for p, _ in done), sum(t for _, t in done)


def cpu_baseline(batch, budget_s):
    """The oracle as it stands on the host's cores, two legs of `budget_s` seconds
    each over the batch's (seq, head) pairs, BLAS limited to one thread per call: one
    thread in this process, then one worker process per available core (at most
    CPU_POOL_LIMIT).  Under a profiler that preloads itself into every process, the
    multi-core leg is skipped (its workers would each open the GPU)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from paged_kv_cache_414_amd import metrics

    cores_available = len(os.sched_getaffinity(0))
    blas_default = max([int(i.get("num_threads", 1)) for i in threadpool_info()
                        if i.get("user_api") == "blas"] or [1])
    per_token = metrics.kv_bytes_per_token(1, 1, batch.head_dim, batch.q.itemsize)
    h_count = batch.num_heads
    with threadpool_limits(limits=1):
        t0 = time.time()
        pairs1, tokens1 = _oracle_pairs(batch, budget_s, 0, 1, t0)
        el1 = time.time() - t0
    gbps1 = metrics.gbps(per_token * tokens1, el1)
    single = {"value": round(gbps1, 4), "unit": "GB/s", "cores": 1,
              "seq_steps_per_s": round(pairs1 / h_count / el1, 4)}
    workers = max(1, min(cores_available, CPU_POOL_LIMIT))
    profiled = "rocprof" in os.environ.get("LD_PRELOAD", "")
    if workers > 1 and not profiled:
        pairsn, tokensn = _multi_core_leg(batch, budget_s, workers)
        gbpsn = metrics.gbps(per_token * tokensn, budget_s)
        multi = (f"{workers} worker processes {pairsn} pairs ({tokensn} tokens, {budget_s:.1f} s); ")
    else:
        workers, pairsn, tokensn, gbpsn, multi = 1, pairs1, tokens1, gbps1, ""
    return {
        "value": round(gbpsn, 4),
        "unit": "GB/s",
        "cores": workers,
        "cores_available": cores_available,
        "cores_used": workers,
        "blas_threads_default": blas_default,
        "blas_threads_per_call": 1,
        "kind": "oracle",
        "sample": (f"the batch's (seq, head) pairs in order, repeating the batch, fp64 numpy: "
                   f"{multi}1 thread {pairs1} pairs ({tokens1} tokens, {el1:.1f} s)"),
        "seq_steps_per_s": round(pairsn / h_count / (budget_s if workers > 1 else el1), 4),
        "single_thread": single,
    }


def run_mix(cls_name, seed, torch, args, **kw):
    """A step mix, each step one call of the native decode-step executor: wall-clock
    seq-steps/s (host block manager, the per-step staging and the launches included;
    synthetic inputs staged in HBM beforehand) of a second, warm run of the whole mix
    (the first run is reported beside it), and the last step's decode re-timed alone
    (the kernel time of whole steps comes from a rocprofv3 trace of the same runs).
    The same mix driven step by step from Python (the same native block manager and
    kernels, one binding call per operation) is timed the same way."""
    from paged_kv_cache_414_amd import metrics, steps

    cls = getattr(steps, cls_name)
    log(args, f"step mix {cls_name} {kw}")
    first = cls(seed=seed, native=True, **kw)
    first.prepare()  # every step's synthetic inputs drawn and placed in HBM, once

    def wall_run(mix):
        mix._inputs = first._inputs
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        rows = 0
        for k in range(mix.steps):
            rows += mix.run_step(k)
        torch.cuda.synchronize()
        return rows / (time.perf_counter() - t0), mix

    native_first, _ = wall_run(first)
    native_warm, mix = wall_run(cls(seed=seed, native=True, **kw))
    ms = time_launches(mix.decode_again, 50, torch)
    ctx = mix.last_context_lens()
    kv = mix.kv_bytes(ctx)
    py_first, _ = wall_run(cls(seed=seed, native=False, **kw))
    py_warm, _ = wall_run(cls(seed=seed, native=False, **kw))
    return {
        "steps": mix.steps,
        "seq_steps_per_s_wall": round(native_warm, 1),
        "first_run_seq_steps_per_s_wall": round(native_first, 1),
        "driver": "native executor, one pa_step_run per step",
        "python_driver_seq_steps_per_s_wall": round(py_warm, 1),
        "python_driver_first_run_seq_steps_per_s_wall": round(py_first, 1),
        "copy_on_write_pairs": mix.copies_total,
        "last_step_decode_ms": round(ms, 5),
        "last_step_decode_kv_gbps": round(metrics.gbps(kv, ms * 1e-3), 1),
        "last_step_sum_context": int(ctx.sum()),
        "note": "decode GB/s at this size may include Infinity Cache hits (working set < 256 MB)",
    }


def long_context_decode(torch, ops, metrics, args):
    """pa_decode on the long-context batch (8 seqs x 32 heads x 128, block 32,
    contexts U[16384, 32768]): partition pass + log-sum-exp merge."""
    from paged_kv_cache_414_amd import workloads

    log(args, "long-context batch")
    b = workloads.long_context(seed=5, poison=False)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    q, k, v = dev(b.q), dev(b.k_pool), dev(b.v_pool)
    tables, ctx = dev(b.block_tables), dev(b.context_lens)
    out = torch.empty_like(q)
    ws = ops.workspace_for(q, k, b.max_context_len, 0)

    def decode():
        ops.pa_decode(out, q, k, v, tables, ctx, b.scale, b.max_context_len, 0, ws)

    def partitions():
        ops.pa_decode_partitions(out, q, k, v, tables, ctx, b.scale, b.max_context_len, 0, ws)

    for _ in range(5):
        decode()
    n = max(10, args.steps // 4)
    ms = time_launches(decode, n, torch)
    ms_part = time_launches(partitions, n, torch)
    spread = launch_spread(decode, n, torch)
    kv = metrics.decode_kv_bytes(b.context_lens, b.num_heads, b.head_dim, 2)
    del q, k, v, tables, ctx, out, ws
    torch.cuda.empty_cache()
    return {
        "sum_context": int(b.context_lens.sum()),
        "partition_tokens": ops.pa_decode_partition_size(b.num_seqs, b.num_heads, b.block_size,
                                                         b.max_context_len),
        "num_partitions": ops.pa_decode_num_partitions(b.num_seqs, b.num_heads, b.block_size,
                                                       b.max_context_len),
        "decode_ms": round(ms, 5),
        "decode_kv_gbps": round(metrics.gbps(kv, ms * 1e-3), 1),
        "pct_of_hbm_peak": round(100.0 * metrics.gbps(kv, ms * 1e-3) / metrics.HBM_PEAK_GBPS, 2),
        "partition_pass_ms": round(ms_part, 5),
        "reduce_ms": round(ms - ms_part, 5),
        "seq_steps_per_s": round(b.num_seqs / (ms * 1e-3), 1),
        "besides_kv": metrics.side_counts(b.context_lens, b.num_heads, b.head_dim, 2, b.block_tables.shape[1],
                                          ops.pa_decode_num_partitions(b.num_seqs, b.num_heads, b.block_size,
                                                                       b.max_context_len)),
        "decode_launch_ms": spread,
    }


def tiny_fp32_decode(torch, ops, metrics, args):
    """pa_decode on the small fp32 batch (4 seqs x 4 heads x 64, block 16, 64-block
    pool): launch-bound, shown for reference."""
    from paged_kv_cache_414_amd import workloads

    log(args, "tiny fp32 batch")
    b = workloads.tiny_fp32(seed=1, poison=False)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    q, k, v = dev(b.q), dev(b.k_pool), dev(b.v_pool)
    tables, ctx = dev(b.block_tables), dev(b.context_lens)
    out = torch.empty_like(q)
    ws = ops.workspace_for(q, k, b.max_context_len, 0)

    def decode():
        ops.pa_decode(out, q, k, v, tables, ctx, b.scale, b.max_context_len, 0, ws)

    for _ in range(20):
        decode()
    n = max(50, args.steps)
    ms = time_launches(decode, n, torch)
    return {
        "num_seqs": b.num_seqs, "num_heads": b.num_heads, "head_dim": b.head_dim,
        "block_size": b.block_size, "dtype": "f32", "sum_context": int(b.context_lens.sum()),
        "decode_ms": round(ms, 5),
        "seq_steps_per_s": round(b.num_seqs / (ms * 1e-3), 1),
        "decode_launch_ms": launch_spread(decode, n, torch),
    }


def shared_prefix_decode(torch, ops, metrics, args):
    """pa_decode against pa_decode_shared_prefix on the shared-prefix mix's last step
    as one batch (8 groups x 8 samples sharing 1024 prompt tokens, 257-271 own tokens
    each): logical bytes count every sequence's tokens, unique bytes count a shared
    block once."""
    from paged_kv_cache_414_amd import workloads

    log(args, "shared-prefix batch")
    b = workloads.shared_prefix_decode(seed=4, poison=False)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    q, k, v = dev(b.q), dev(b.k_pool), dev(b.v_pool)
    tables, ctx = dev(b.block_tables), dev(b.context_lens)
    starts, prefix = dev(b.group_starts), dev(b.prefix_lens)
    out = torch.empty_like(q)
    ws = ops.workspace_for(q, k, b.max_context_len, 0)
    largest = int(np.diff(b.group_starts).max())
    ws2 = ops.shared_prefix_workspace_for(q, k, b.num_groups, b.max_prefix_len, b.max_suffix_len,
                                          max_group_size=largest)

    def plain():
        ops.pa_decode(out, q, k, v, tables, ctx, b.scale, b.max_context_len, 0, ws)

    def shared():
        ops.pa_decode_shared_prefix(out, q, k, v, tables, ctx, starts, prefix, b.scale,
                                    b.max_prefix_len, b.max_suffix_len, workspace=ws2,
                                    max_group_size=largest)

    for _ in range(10):
        plain()
        shared()
    n = max(20, args.steps)
    ms_plain = time_launches(plain, n, torch)
    ms_shared = time_launches(shared, n, torch)
    per_token = metrics.kv_bytes_per_token(1, b.num_heads, b.head_dim, 2)
    logical = metrics.decode_kv_bytes(b.context_lens, b.num_heads, b.head_dim, 2)
    first = b.group_starts[:-1]
    unique = per_token * int((b.context_lens - b.prefix_lens).sum() + b.prefix_lens[first].sum())
    return {
        "groups": b.num_groups, "seqs": b.num_seqs, "prefix_tokens": b.max_prefix_len,
        "logical_kv_bytes": logical, "unique_kv_bytes": unique,
        "pa_decode_ms": round(ms_plain, 5),
        "pa_decode_shared_prefix_ms": round(ms_shared, 5),
        "speedup": round(ms_plain / ms_shared, 3),
        "shared_unique_kv_gbps": round(metrics.gbps(unique, ms_shared * 1e-3), 1),
        "shared_logical_kv_gbps": round(metrics.gbps(logical, ms_shared * 1e-3), 1),
        "note": "pa_decode re-reads each shared block per sample (partly from cache)",
    }


def graph_step(torch, ops, metrics, args):
    """Small-batch decode steps, launched directly vs replayed from a recorded graph:
    wall-clock per step over back-to-back steps on fixed inputs (launch overhead
    isolated), for the two-launch step (pa_cache_append + pa_decode) and for the
    single pa_decode_append launch."""
    from paged_kv_cache_414_amd import blocks, graphs, workloads

    log(args, "graph-captured step")
    rows = []
    for s_count in (1, 8, 64):
        b = workloads.make_static_batch("graph_step", seed=11, num_seqs=s_count, num_heads=32,
                                        head_dim=128, block_size=16, ctx_low=64, ctx_high=512,
                                        dtype=np.float16, pool_slack=1.2, max_blocks_per_seq=33,
                                        poison=False)
        k = torch.from_numpy(b.k_pool).cuda()
        v = torch.from_numpy(b.v_pool).cuda()
        g = graphs.DecodeStepGraph(k, v, s_count, 33, 33 * 16, b.scale)
        gf = graphs.DecodeStepGraph(k, v, s_count, 33, 33 * 16, b.scale, fused=True)
        for gg in (g, gf):
            gg.q.copy_(torch.from_numpy(b.q))
            gg.new_k.copy_(torch.from_numpy(b.q))
            gg.new_v.copy_(torch.from_numpy(b.q))
            gg.block_tables.copy_(torch.from_numpy(b.block_tables))
            gg.context_lens.copy_(torch.from_numpy(b.context_lens))
        # the two-launch step appends at the newest position too (the fused one
        # always does): both rewrite the same slot with the same row every step
        pos = b.context_lens.astype(np.int64) - 1
        g.slots.copy_(torch.from_numpy(
            blocks.slots_for_positions(b.block_tables, pos, 16).astype(np.int32)))

        def wall(fn, n=300):
            for _ in range(20):
                fn()
            torch.cuda.synchronize()
            time.sleep(0.05)  # an idle stretch marks the start of each timed run in a trace
            t0 = time.perf_counter()
            for _ in range(n):
                fn()
            torch.cuda.synchronize()
            return (time.perf_counter() - t0) / n * 1e6

        eager_us = wall(g.run_eager)
        graph_us = wall(g.replay)
        gpu_ms = time_launches(g.replay, 100, torch)
        fused_us = wall(gf.run_eager)
        fused_graph_us = wall(gf.replay)
        fused_gpu_ms = time_launches(gf.run_eager, 100, torch)
        rows.append({"num_seqs": s_count, "sum_context": int(b.context_lens.sum()),
                     "eager_us_per_step": round(eager_us, 2),
                     "graph_us_per_step": round(graph_us, 2),
                     "speedup": round(eager_us / graph_us, 3),
                     "gpu_us_per_step": round(gpu_ms * 1e3, 2),
                     "fused_eager_us_per_step": round(fused_us, 2),
                     "fused_graph_us_per_step": round(fused_graph_us, 2),
                     "fused_gpu_us_per_step": round(fused_gpu_ms * 1e3, 2),
                     "fused_speedup": round(eager_us / fused_us, 3)})
        del g, gf, k, v
        torch.cuda.empty_cache()
    return rows


def swap_throughput(torch, ops, args, pairs=2048):
    """pa_swap_blocks of ``pairs`` Llama-shaped blocks (32 heads x 16 x 128 fp16:
    128 KiB of K and 128 KiB of V each) from the GPU pool to a pinned host pool and
    back: bytes moved / time, each direction."""
    log(args, "block swap")
    shape = (pairs, 32, 16, 128)
    gk = torch.randn(shape, dtype=torch.float16, device="cuda")
    gv = torch.randn(shape, dtype=torch.float16, device="cuda")
    hk = torch.empty(shape, dtype=torch.float16, pin_memory=True)
    hv = torch.empty(shape, dtype=torch.float16, pin_memory=True)
    ids = torch.randperm(pairs, generator=torch.Generator().manual_seed(3))
    out_pairs = torch.stack([torch.arange(pairs), ids], dim=1).to(torch.int32).cuda()
    in_pairs = torch.stack([ids, torch.arange(pairs)], dim=1).to(torch.int32).cuda()
    moved = 2 * pairs * 32 * 16 * 128 * 2
    res = {"pairs": pairs, "bytes_each_way": moved}
    for name, fn in (("out", lambda: ops.pa_swap_blocks(hk, hv, gk, gv, out_pairs)),
                     ("in", lambda: ops.pa_swap_blocks(gk, gv, hk, hv, in_pairs))):
        fn()
        ms = time_launches(fn, 5, torch)
        res[f"swap_{name}_ms"] = round(ms, 4)
        res[f"swap_{name}_gbps"] = round(moved / (ms * 1e-3) / 1e9, 2)
    del gk, gv, hk, hv
    torch.cuda.empty_cache()
    return res


def append_copy_throughput(torch, ops, metrics, args):
    """pa_cache_append and pa_block_copy alone, Llama-shaped rows and blocks (32 heads
    x 128, block 16, fp16), on the GPU pool: average time per launch over back-to-back
    launches and bytes read + written per second against HBM peak.

    append: the 96 rows of one decode step (latency-sized), and 4,096 prompt rows
    filling 256 whole blocks scattered over the pool (bandwidth-sized; the launches
    cycle through 6 sets of rows and blocks, 400 MB in all, so that no launch finds the
    previous one's rows in the 256 MB Infinity Cache).  copy: the 56 copy-on-write
    pairs of the shared-prefix step (8 groups x 7 copies), and 2,048 pairs (512 MiB of
    K and V read and written)."""
    log(args, "append and block copy")
    heads, bs, d = 32, 16, 128
    nb = 8192
    gen = torch.Generator(device="cuda").manual_seed(5)
    kc = torch.randn((nb, heads, bs, d), dtype=torch.float16, device="cuda", generator=gen)
    vc = torch.randn((nb, heads, bs, d), dtype=torch.float16, device="cuda", generator=gen)
    rng = np.random.default_rng([args.seed, 11])
    ids = rng.permutation(nb).astype(np.int64)
    n = max(50, args.steps)
    res = {}
    for name, tokens, sets in (("append_step_rows", 96, 1), ("append_prompt_rows", 4096, 6)):
        args_of_set = []
        for j in range(sets):
            if tokens <= 96:  # one row at the end of each of 96 blocks
                slots = ids[:tokens] * bs + (bs - 1)
            else:             # whole blocks, token t at offset t % bs of block t // bs
                t = np.arange(tokens)
                slots = ids[j * (tokens // bs) + t // bs] * bs + t % bs
            slots_d = torch.from_numpy(slots.astype(np.int32)).cuda()
            nk = torch.randn((tokens, heads, d), dtype=torch.float16, device="cuda", generator=gen)
            nv = torch.randn((tokens, heads, d), dtype=torch.float16, device="cuda", generator=gen)
            args_of_set.append((nk, nv, slots_d))
        turn = [0]

        def fn():
            nk, nv, slots_d = args_of_set[turn[0] % sets]
            turn[0] += 1
            ops.pa_cache_append(kc, vc, nk, nv, slots_d)

        for _ in range(10):
            fn()
        ms = time_launches(fn, n, torch)
        moved = metrics.append_bytes(tokens, heads, d, 2)
        res[name] = {"rows": tokens, "us": round(ms * 1e3, 2), "bytes": moved,
                     "gbps": round(metrics.gbps(moved, ms * 1e-3), 1),
                     "pct_of_hbm_peak": round(100.0 * metrics.gbps(moved, ms * 1e-3) /
                                              metrics.HBM_PEAK_GBPS, 1)}
    for name, pairs in (("copy_on_write_pairs", 56), ("copy_large", 2048)):
        src = ids[:pairs]
        dst = ids[nb - pairs:]
        pairs_d = torch.from_numpy(np.stack([src, dst], axis=1).astype(np.int32)).cuda()
        fn = lambda: ops.pa_block_copy(kc, vc, pairs_d)  # noqa: E731
        for _ in range(5):
            fn()
        ms = time_launches(fn, n if pairs < 1024 else 20, torch)
        moved = metrics.block_copy_bytes(pairs, heads, bs, d, 2)
        res[name] = {"pairs": pairs, "us": round(ms * 1e3, 2), "bytes": moved,
                     "gbps": round(metrics.gbps(moved, ms * 1e-3), 1),
                     "pct_of_hbm_peak": round(100.0 * metrics.gbps(moved, ms * 1e-3) /
                                              metrics.HBM_PEAK_GBPS, 1)}
    res["note"] = ("bytes = K and V rows read plus written; the step rows and the 56 pairs "
                   "are latency-sized (a few MB), so their GB/s is not a bandwidth figure")
    del kc, vc
    torch.cuda.empty_cache()
    return res


def shared_prefix_groups(torch, ops, metrics, args):
    """pa_decode against pa_decode_shared_prefix for other group layouts (32 heads, fp16;
    each member holds 200-330 tokens of its own after the shared prefix): many small
    groups, one group of 64 sharing a long prompt and one group of 256 (a prompt shared
    by the whole batch), at head dim 128 and block 16; and the small groups at head dim
    256, and with blocks of 8 tokens and a prefix of an odd number of blocks."""
    from paged_kv_cache_414_amd import workloads

    log(args, "shared-prefix group layouts")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    rows = []
    # (group sizes, shared tokens, head dim, block size)
    for sizes, prefix_tokens, hd, bs in (([8] * 8, 1024, 128, 16), ([64], 2048, 128, 16),
                                         ([256], 512, 128, 16), ([8] * 8, 1024, 256, 16),
                                         ([8] * 8, 1032, 128, 8)):
        b = workloads.make_shared_prefix_batch("groups", seed=3, group_sizes=sizes, num_heads=32,
                                               head_dim=hd, block_size=bs,
                                               prefix_blocks_low=prefix_tokens // bs,
                                               prefix_blocks_high=prefix_tokens // bs, suffix_low=200,
                                               suffix_high=330, poison=False)
        q, k, v = dev(b.q), dev(b.k_pool), dev(b.v_pool)
        tables, ctx = dev(b.block_tables), dev(b.context_lens)
        starts, prefix = dev(b.group_starts), dev(b.prefix_lens)
        out = torch.empty_like(q)
        ws = ops.workspace_for(q, k, b.max_context_len, 0)
        ws2 = ops.shared_prefix_workspace_for(q, k, b.num_groups, b.max_prefix_len,
                                              b.max_suffix_len, max_group_size=max(sizes))

        def plain():
            ops.pa_decode(out, q, k, v, tables, ctx, b.scale, b.max_context_len, 0, ws)

        def shared():
            ops.pa_decode_shared_prefix(out, q, k, v, tables, ctx, starts, prefix, b.scale,
                                        b.max_prefix_len, b.max_suffix_len, workspace=ws2,
                                        max_group_size=max(sizes))

        for _ in range(10):
            plain()
            shared()
        n = max(20, args.steps // 2)
        ms_plain = time_launches(plain, n, torch)
        ms_shared = time_launches(shared, n, torch)
        per_token = metrics.kv_bytes_per_token(1, b.num_heads, b.head_dim, 2)
        unique = per_token * int((b.context_lens - b.prefix_lens).sum() +
                                 b.prefix_lens[b.group_starts[:-1]].sum())
        rows.append({"groups": f"{len(sizes)} x {sizes[0]}", "prefix_tokens": prefix_tokens,
                     "head_dim": hd, "block_size": bs,
                     "pa_decode_ms": round(ms_plain, 5),
                     "pa_decode_shared_prefix_ms": round(ms_shared, 5),
                     "speedup": round(ms_plain / ms_shared, 3),
                     "shared_unique_kv_gbps": round(metrics.gbps(unique, ms_shared * 1e-3), 1)})
        del q, k, v, tables, ctx, starts, prefix, out, ws, ws2
        torch.cuda.empty_cache()
    return rows


def copy_probe(torch, ops, metrics, pairs=1024):
    """One pa_block_copy of ``pairs`` blocks of 32 heads x 16 x 128 fp16 (128 KiB per
    block for K and for V): a plain copy of known size, run once, whose memory
    counters calibrate those of the decode kernel."""
    block = (32, 16, 128)
    kc = torch.zeros((2 * pairs, *block), dtype=torch.float16, device="cuda")
    vc = torch.zeros_like(kc)
    pairs_d = torch.stack([torch.arange(pairs), torch.arange(pairs, 2 * pairs)], dim=1)
    pairs_d = pairs_d.to(torch.int32).cuda()
    torch.cuda.synchronize()
    ops.pa_block_copy(kc, vc, pairs_d)
    torch.cuda.synchronize()
    moved = metrics.block_copy_bytes(pairs, *block[:2], block[2], 2) // 2
    return {"kernel": "block_copy_kernel", "read_bytes": moved, "write_bytes": moved}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(across GPUs the decode path would shard by sequence or by head, with no exchange "
              "between them)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from paged_kv_cache_414_amd import blocks, metrics, ops, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.graph_only:
        print(json.dumps({"graph_step": graph_step(torch, ops, metrics, args)}), flush=True)
        return
    if args.sweep:
        from paged_kv_cache_414_amd import sweep
        log(args, "block-size and head-dim sweep")
        print(json.dumps(sweep.run(seed=args.seed, steps=min(args.steps, 50))), flush=True)
        return

    log(args, "generating the llama7b_decode batch")
    batch = workloads.llama7b_decode(seed=args.seed, poison=False)
    s_count, h_count, d = batch.q.shape
    bs = batch.block_size
    ctx = batch.context_lens
    max_ctx = batch.max_context_len
    positions = ctx.astype(np.int64) - 1  # each sequence's newest token
    slots = blocks.slots_for_positions(batch.block_tables, positions, bs)
    rng = np.random.default_rng([args.seed, 7])
    new_k = workloads.normal(rng, (s_count, h_count, d), batch.dtype)
    new_v = workloads.normal(rng, (s_count, h_count, d), batch.dtype)

    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    q, kc, vc = dev(batch.q), dev(batch.k_pool), dev(batch.v_pool)
    tables, ctx_d, slots_d = dev(batch.block_tables), dev(ctx), dev(slots)
    nk, nv = dev(new_k), dev(new_v)
    out = torch.empty_like(q)
    part = ops.pa_decode_partition_size(s_count, h_count, bs, max_ctx, args.partition)
    n_parts = ops.pa_decode_num_partitions(s_count, h_count, bs, max_ctx, args.partition)
    ws = ops.workspace_for(q, kc, max_ctx, args.partition)

    def step():  # one launch: the 96 new rows appended inside the decode
        ops.pa_decode_append(out, q, kc, vc, nk, nv, tables, ctx_d, batch.scale, max_ctx,
                             args.partition, ws)

    def two_launch_step():  # the same work as two calls
        ops.pa_cache_append(kc, vc, nk, nv, slots_d)
        ops.pa_decode(out, q, kc, vc, tables, ctx_d, batch.scale, max_ctx, args.partition, ws)

    def partitions_only():
        ops.pa_decode_partitions(out, q, kc, vc, tables, ctx_d, batch.scale, max_ctx,
                                 args.partition, ws)

    def decode_only():
        ops.pa_decode(out, q, kc, vc, tables, ctx_d, batch.scale, max_ctx, args.partition, ws)

    log(args, f"warmup {args.warmup} steps (P={part}, NP={n_parts})")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    log(args, f"timing {args.steps} steps")
    ms_step = time_launches(step, args.steps, torch)
    log(args, "timing the partition pass alone")
    for _ in range(args.warmup):
        partitions_only()
    ms_part = time_launches(partitions_only, args.steps, torch)
    ms_decode = time_launches(decode_only, args.steps, torch)
    ms_two = time_launches(two_launch_step, args.steps, torch)
    decode_spread = launch_spread(decode_only, args.steps, torch)

    kv = metrics.decode_kv_bytes(ctx, h_count, d, batch.q.itemsize)
    value = metrics.gbps(kv, ms_step * 1e-3)
    waves = ops.pa_decode_waves(s_count, h_count, d, bs, max_ctx, args.partition)
    # the step's launch reads every live K/V row once (the 96 new rows from new_key /
    # new_value, counted in kv since the contexts count them) and writes the 96 new rows
    launch_bytes = kv + metrics.fused_append_bytes(s_count, h_count, d, batch.q.itemsize)
    achieved = metrics.gbps(launch_bytes, ms_step * 1e-3)
    achieved_alone = metrics.gbps(kv, ms_part * 1e-3)
    record = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "accumulate": "f32",
        "data": "synthetic",
        "config": {
            "workload": "llama7b_decode",
            "num_seqs": s_count, "num_heads": h_count, "head_dim": d, "block_size": bs,
            "context_lens": "uniform [300, 2048]", "sum_context": int(ctx.sum()),
            "max_context": max_ctx, "num_blocks": batch.num_blocks,
            "partition_tokens": part, "num_partitions": n_parts, "seed": args.seed,
            "step": "pa_decode_append: the 96 new rows appended inside the decode launch",
        },
        "pct_of_hbm_peak": round(100.0 * value / metrics.HBM_PEAK_GBPS, 2),
        "seq_steps_per_s": round(s_count / (ms_step * 1e-3), 1),
        "decode_ms": round(ms_decode, 5),
        "decode_kv_gbps": round(metrics.gbps(kv, ms_decode * 1e-3), 2),
        "decode_launch_ms": decode_spread,
        "two_launch_step": {"calls": "pa_cache_append (96 rows) + pa_decode (the same work)",
                            "ms": round(ms_two, 5),
                            "kv_gbps": round(metrics.gbps(kv, ms_two * 1e-3), 2)},
        "decode_partition_pass_alone": {"ms": round(ms_part, 5),
                                        "kv_gbps": round(achieved_alone, 2),
                                        "frac": round(achieved_alone / metrics.HBM_PEAK_GBPS, 4)},
        "kv_bytes_per_step": kv,
        "besides_kv": metrics.side_counts(ctx, h_count, d, batch.q.itemsize, batch.block_tables.shape[1],
                                          n_parts),
        "roofline": {
            "kernel": (f"decode_partitions_kernel<f16, 128, 16>, {waves} waves per workgroup, "
                       "with the append fused (pa_decode_append)"),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": metrics.HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / metrics.HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(args.seed, part),
            "avg_launch_ms": round(ms_step, 5),
            "algorithmic_bytes_per_launch": launch_bytes,
        },
    }
    if args.extras:
        record["long_context"] = long_context_decode(torch, ops, metrics, args)
        record["tiny_fp32"] = tiny_fp32_decode(torch, ops, metrics, args)
        record["shared_prefix_decode"] = shared_prefix_decode(torch, ops, metrics, args)
        record["shared_prefix_groups"] = shared_prefix_groups(torch, ops, metrics, args)
        if args.graph:
            record["graph_step"] = graph_step(torch, ops, metrics, args)
        record["block_swap"] = swap_throughput(torch, ops, args)
        record["append_and_copy"] = append_copy_throughput(torch, ops, metrics, args)
    if args.mixes:
        record["step_mixes"] = {
            "continuous_batching": run_mix("ContinuousBatching", 3, torch, args),
            "shared_prefix_cow": run_mix("SharedPrefix", 4, torch, args),
            "shared_prefix_cow_shared_decode": run_mix("SharedPrefix", 4, torch, args,
                                                       shared_decode=True),
        }
    if args.copy_probe:
        record["copy_probe"] = copy_probe(torch, ops, metrics)
    if args.cpu_seconds > 0:
        log(args, f"CPU oracle baseline ({args.cpu_seconds:.0f} s per leg)")
        record["cpu_baseline"] = cpu_baseline(batch, args.cpu_seconds)
    else:
        record["cpu_baseline"] = None
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
