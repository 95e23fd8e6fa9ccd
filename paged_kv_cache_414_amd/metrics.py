"""Algorithmic byte accounting for the paged decode path.

The per-token KV footprint is 2 (K and V) x layers x heads x head_dim x bytes per
element, the product the page "vLLM基础：架构、推理流程与关键组件" (vLLM basics) uses
in §2.3 (about 1 GB for a 2048-token Llama-7B-shaped sequence in fp16) and in the
§2.5 case study (about 1.2 GB for 8 requests of 300 tokens).

What one decode call must move from HBM, at the least, is every live token's K and
V row of every head once: 2 * sum(context_lens) * heads * head_dim * element bytes.
Padding slots of partly filled blocks, the block table, q and the output are not
counted.
"""

from __future__ import annotations

import numpy as np

# MI355X HBM3E peak bandwidth (AMD specification), GB/s (1 GB = 1e9 bytes).
HBM_PEAK_GBPS = 8000.0


def kv_bytes_per_token(layers: int, heads: int, head_dim: int, elem_bytes: int) -> int:
    return 2 * int(layers) * int(heads) * int(head_dim) * int(elem_bytes)


def kv_cache_bytes(tokens: int, seqs: int, layers: int, heads: int, head_dim: int,
                   elem_bytes: int) -> int:
    return int(seqs) * int(tokens) * kv_bytes_per_token(layers, heads, head_dim, elem_bytes)


def decode_kv_bytes(context_lens, heads: int, head_dim: int, elem_bytes: int) -> int:
    """Algorithmic HBM bytes of one decode call over one layer."""
    total_tokens = int(np.asarray(context_lens, dtype=np.int64).sum())
    return kv_bytes_per_token(1, heads, head_dim, elem_bytes) * total_tokens


def decode_flops(context_lens, heads: int, head_dim: int) -> int:
    """Multiply-adds of QK and PV counted as 2 flops each."""
    total_tokens = int(np.asarray(context_lens, dtype=np.int64).sum())
    return 4 * total_tokens * int(heads) * int(head_dim)


def side_counts(context_lens, heads: int, head_dim: int, elem_bytes: int,
                max_blocks_per_seq: int, num_partitions: int) -> dict:
    """What a decode call moves or computes besides the K and V rows: q read and the
    output written (S x H x D elements each), the block table and context lengths
    read (int32), the partition states written and read back when the call splits the
    contexts (m, l and o in float32 per (sequence, head, partition)), the flops of
    :func:`decode_flops` and one exponential per (token, head)."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    s, h, d = len(ctx), int(heads), int(head_dim)
    total = int(ctx.sum())
    np_ = int(num_partitions)
    return {
        "q_bytes": s * h * d * int(elem_bytes),
        "out_bytes": s * h * d * int(elem_bytes),
        "table_bytes": s * int(max_blocks_per_seq) * 4 + s * 4,
        "workspace_bytes": 2 * s * h * np_ * (d + 2) * 4 if np_ > 1 else 0,
        "flops": decode_flops(ctx, h, d),
        "transcendentals": total * h,
    }


def append_bytes(num_tokens: int, heads: int, head_dim: int, elem_bytes: int) -> int:
    """Read and write of the appended K and V rows."""
    return 2 * 2 * int(num_tokens) * int(heads) * int(head_dim) * int(elem_bytes)


def fused_append_bytes(num_tokens: int, heads: int, head_dim: int, elem_bytes: int) -> int:
    """What appending inside the decode launch adds to the decode's bytes: the new K
    and V rows written.  Their read is already among the decode's live rows, since the
    contexts count the new tokens."""
    return 2 * int(num_tokens) * int(heads) * int(head_dim) * int(elem_bytes)


def block_copy_bytes(num_pairs: int, heads: int, block_size: int, head_dim: int,
                     elem_bytes: int) -> int:
    """Read and write of K and V of every copied block."""
    return 2 * 2 * int(num_pairs) * int(heads) * int(block_size) * int(head_dim) * int(elem_bytes)


def gbps(nbytes: float, seconds: float) -> float:
    return nbytes / seconds / 1e9
