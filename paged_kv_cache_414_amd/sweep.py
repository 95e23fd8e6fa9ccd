"""Block-size and head-dim sweep of pa_decode on one GPU.

"Reading the vLLM source ..." §2.3 weighs the block size: small blocks cost
bookkeeping (longer block tables, more allocations), large blocks waste the unused
tail of each sequence's last block (fragmentation), 16 tokens being the default.
This sweep measures both sides on MI355X for the Llama-7B-shaped batch (96
sequences, contexts uniform in [300, 2048], fp16): for every block size it reports
the decode time and KV GB/s, the padding waste of the last blocks, the block-table
entries per sequence, and the host block manager's time to reserve one token per
sequence (one decode step's bookkeeping).  A second sweep varies the head dim at
block size 16 (32 heads), and a third fp32 K/V and q against fp16 (block size 16,
32 heads x 128).

Inputs: the contexts and the scattered block ids are drawn with numpy (PCG64,
seeded); the K/V pools, which only need to exist for timing, are filled on the GPU
(torch's seeded normal generator).  Parity for every (head dim, block size) is
covered by the tests, not here.

    python bench.py --sweep          # one JSON line
"""

from __future__ import annotations

import time

import numpy as np
import torch

from . import blocks, metrics, ops

BLOCK_SIZES = (8, 16, 32, 64, 128, 256)
HEAD_DIMS = (64, 80, 96, 128, 256)


def _time(fn, n: int) -> float:
    for _ in range(5):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(n):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / n


def _case(seed: int, ctx: np.ndarray, num_heads: int, head_dim: int, block_size: int,
          steps: int, dtype: torch.dtype = torch.float16) -> dict:
    rng = np.random.default_rng([seed, block_size, head_dim])
    n_blk = -(-ctx.astype(np.int64) // block_size)
    needed = int(n_blk.sum())
    num_blocks = int(np.ceil(1.1 * needed))
    perm = rng.permutation(num_blocks).astype(np.int32)
    mb = int(n_blk.max())
    tables = np.zeros((ctx.size, mb), dtype=np.int32)
    cursor = 0
    for s, n in enumerate(n_blk):
        tables[s, :n] = perm[cursor:cursor + n]
        cursor += n
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed * 1000 + block_size + head_dim)
    shape = (num_blocks, num_heads, block_size, head_dim)
    k = torch.randn(shape, dtype=dtype, device="cuda", generator=gen)
    v = torch.randn(shape, dtype=dtype, device="cuda", generator=gen)
    q = torch.randn((ctx.size, num_heads, head_dim), dtype=dtype, device="cuda",
                    generator=gen)
    out = torch.empty_like(q)
    tables_d = torch.from_numpy(tables).cuda()
    ctx_d = torch.from_numpy(ctx).cuda()
    max_ctx = int(ctx.max())
    ws = ops.workspace_for(q, k, max_ctx, 0)
    ms = _time(lambda: ops.pa_decode(out, q, k, v, tables_d, ctx_d, 1.0 / np.sqrt(head_dim),
                                     max_ctx, 0, ws), steps)
    kv = metrics.decode_kv_bytes(ctx, num_heads, head_dim, q.element_size())
    del k, v, q, out, ws
    torch.cuda.empty_cache()
    allocated = int(n_blk.sum()) * block_size
    # host bookkeeping of one step: reserve the next token of every sequence
    mgr = blocks.BlockManager(num_blocks + ctx.size, block_size, seed=seed + 1)
    for s, c in enumerate(ctx):
        mgr.add_sequence(s, int(c))
    ids = np.arange(ctx.size, dtype=np.int64)
    t0 = time.perf_counter()
    rounds = 50
    for _ in range(rounds):
        mgr.append_slots(ids)
        mgr.block_tables(ids, mb + rounds)
    host_us = (time.perf_counter() - t0) / rounds * 1e6
    return {
        "block_size": block_size, "head_dim": head_dim, "num_heads": num_heads,
        "dtype": "f32" if dtype == torch.float32 else "f16",
        "partition_tokens": ops.pa_decode_partition_size(ctx.size, num_heads, block_size, max_ctx),
        "decode_ms": round(ms, 5),
        "kv_gbps": round(metrics.gbps(kv, ms * 1e-3), 1),
        "pct_of_hbm_peak": round(100.0 * metrics.gbps(kv, ms * 1e-3) / metrics.HBM_PEAK_GBPS, 2),
        "padding_waste_pct": round(100.0 * (allocated - int(ctx.sum())) / allocated, 3),
        "table_entries_per_seq": round(float(n_blk.mean()), 1),
        "host_step_us": round(host_us, 1),
    }


def run(seed: int = 2, steps: int = 50) -> dict:
    rng = np.random.default_rng(seed)
    ctx = rng.integers(300, 2049, size=96).astype(np.int32)
    by_block = [_case(seed, ctx, 32, 128, bs, steps) for bs in BLOCK_SIZES]
    by_dim = [_case(seed, ctx, 32, d, 16, steps) for d in HEAD_DIMS]
    by_dtype = [_case(seed, ctx, 32, 128, 16, steps, dtype)
                for dtype in (torch.float16, torch.float32)]
    return {
        "metric": "pa_decode KV GB/s by block size and head dim (1 GPU)",
        "workload": "96 seqs, contexts U[300, 2048], fp16 K/V and q (fp32 in the dtype "
                    "sweep), fp32 accumulate",
        "sum_context": int(ctx.sum()),
        "block_size_sweep": by_block,
        "head_dim_sweep": by_dim,
        "dtype_sweep": by_dtype,
        "host_step_us_note": "native block manager: reserve 96 slots + build the block "
                             "tables, per step, on the host",
    }
