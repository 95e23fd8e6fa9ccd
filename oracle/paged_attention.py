"""CPU oracle for the paged-attention decode path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module.  It shares no code with the HIP path and
imports nothing from the product package.

Pages cited (by title and section):
  [Reading vLLM]   "啃透vLLM源码：从PagedAttention到连续批处理，大模型推理加速24倍的秘密"
                   (Reading the vLLM source: from PagedAttention to continuous batching)
  [vLLM basics]    "vLLM基础：架构、推理流程与关键组件"
                   (vLLM basics: architecture, inference flow and key components)
  [vLLM analysis]  "VLLM源码解析：高效大规模语言模型推理的技术实现"
                   (vLLM source analysis: technical implementation of efficient inference)

What the method computes, and therefore what this oracle computes:
  * The KV cache of a sequence is cut into fixed-size blocks (16 tokens by default);
    logical block i of a sequence lives in whatever physical block its block table
    names, and physical blocks may sit anywhere in the pool ([Reading vLLM] §2.2;
    [vLLM basics] §2.3, block table).
  * Attention for the newest token reads the query, the key and value caches and the
    physical block indices of its sequence ([vLLM analysis] "设计原理" / design
    principles, the attention_forward sketch).
  * Paging changes where the numbers live, not what attention computes, so the
    result is ordinary single-query softmax attention over the sequence's tokens in
    logical order.  The oracle writes that definition out: gather the blocks through
    the table into contiguous K and V, then max-subtracted softmax of the scaled dot
    products, then the weighted sum of V rows.  Everything is float64 from the exact
    upcast of the stored values.
  * New tokens are written into the slot their position maps to ([Reading vLLM]
    §2.2, LogicalTokenBlock.append_tokens: a block fills slot by slot).
  * Blocks may be shared by reference count; a sharer that has to write gets its own
    copy of the block first ([Reading vLLM] §2.2; [vLLM basics] §2.3, copy-on-write).
    Copying a block copies all of its K and V bytes.

Readings where the pages are silent (each is listed with its reason in the design
notes of the repository):
  * Pool layout [num_blocks, heads, block_size, head_dim] for K and V alike.
  * slot = physical_block * block_size + offset_in_block; a negative slot is skipped.
  * A context of length 0 yields a zero output.
  * Block-copy pairs act as if every source were read before any destination is
    written; destinations are distinct and never a source.

Partition states (used to check the split-context pass in isolation): for the tokens
t of one partition, m = max_t z_t, l = sum_t exp(z_t - m), o = sum_t exp(z_t - m) v_t,
with z_t = scale * <q, k_t>.  Merging partitions by the log-sum-exp rule gives back
the unsplit attention (Milakov & Gimelshein 2018, "Online normalizer calculation for
softmax").
"""

from __future__ import annotations

import math

import numpy as np


# ----------------------------------------------------------------------------------
# addressing through the block table ([vLLM basics] §2.3; [Reading vLLM] §2.2)
# ----------------------------------------------------------------------------------

def token_location(block_table_row, position: int, block_size: int) -> tuple[int, int]:
    """Physical (block, offset) that holds logical token ``position`` of a sequence."""
    logical_block, offset = divmod(int(position), int(block_size))
    return int(block_table_row[logical_block]), offset


def slot_of(block_table_row, position: int, block_size: int) -> int:
    """Flat slot index of logical token ``position``: block * block_size + offset."""
    block, offset = token_location(block_table_row, position, block_size)
    return block * int(block_size) + offset


def gather_head(pool: np.ndarray, block_table_row, context_len: int,
                head: int) -> np.ndarray:
    """Contiguous [context_len, D] float64 rows of one head of one sequence."""
    block_size = pool.shape[2]
    rows = np.empty((int(context_len), pool.shape[3]), dtype=np.float64)
    for t in range(int(context_len)):
        b, o = token_location(block_table_row, t, block_size)
        rows[t] = pool[b, head, o, :]
    return rows


def gather_head_fast(pool: np.ndarray, block_table_row, context_len: int,
                     head: int) -> np.ndarray:
    """Same rows as :func:`gather_head`, whole blocks at a time (for large inputs)."""
    block_size = pool.shape[2]
    n_blocks = -(-int(context_len) // block_size)
    ids = np.asarray(block_table_row[:n_blocks], dtype=np.int64)
    rows = pool[ids, head, :, :].reshape(n_blocks * block_size, pool.shape[3])
    return rows[:int(context_len)].astype(np.float64)


# ----------------------------------------------------------------------------------
# decode attention
# ----------------------------------------------------------------------------------

def attention_weights(q_row: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    """Softmax weights of one query over ``keys`` [L, D], max-subtracted."""
    z = float(scale) * (keys @ np.asarray(q_row, dtype=np.float64))
    e = np.exp(z - z.max())
    return e / e.sum()


def decode_one(q_row, k_pool, v_pool, block_table_row, context_len, head, scale,
               fast: bool = True) -> np.ndarray:
    """Attention output [D] (float64) of one (sequence, head)."""
    d = k_pool.shape[3]
    if int(context_len) == 0:
        return np.zeros(d, dtype=np.float64)
    gather = gather_head_fast if fast else gather_head
    keys = gather(k_pool, block_table_row, context_len, head)
    values = gather(v_pool, block_table_row, context_len, head)
    w = attention_weights(q_row, keys, scale)
    return w @ values


def decode(q, k_pool, v_pool, block_tables, context_lens, scale,
           fast: bool = True) -> np.ndarray:
    """Paged decode attention for a batch: float64 [S, H, D].

    q [S, H, D]; pools [NB, H, bs, D]; block_tables [S, MB]; context_lens [S]."""
    s_count, h_count, d = q.shape
    out = np.zeros((s_count, h_count, d), dtype=np.float64)
    for s in range(s_count):
        for h in range(h_count):
            out[s, h] = decode_one(q[s, h], k_pool, v_pool, block_tables[s],
                                   context_lens[s], h, scale, fast=fast)
    return out


# ----------------------------------------------------------------------------------
# split-context partition states and their merge
# ----------------------------------------------------------------------------------

def partition_state(q_row, k_pool, v_pool, block_table_row, context_len, head, scale,
                    start: int, stop: int):
    """(m, l, o) over logical tokens [start, min(stop, context_len)) of one head.

    m = max z_t, l = sum exp(z_t - m), o = sum exp(z_t - m) v_t (natural base)."""
    stop = min(int(stop), int(context_len))
    if stop <= start:
        raise ValueError("empty partition")
    keys = gather_head_fast(k_pool, block_table_row, stop, head)[start:stop]
    values = gather_head_fast(v_pool, block_table_row, stop, head)[start:stop]
    z = float(scale) * (keys @ np.asarray(q_row, dtype=np.float64))
    m = z.max()
    e = np.exp(z - m)
    return float(m), float(e.sum()), e @ values


def merge_partition_states(ms, ls, os_):
    """Log-sum-exp merge of partition states into the normalised output [D]."""
    ms = np.asarray(ms, dtype=np.float64)
    ls = np.asarray(ls, dtype=np.float64)
    os_ = np.asarray(os_, dtype=np.float64)
    top = ms.max()
    f = np.exp(ms - top)
    return (f[:, None] * os_).sum(axis=0) / (f * ls).sum()


# ----------------------------------------------------------------------------------
# brute force: scalar Python, math.exp and math.fsum, tiny inputs only
# ----------------------------------------------------------------------------------

def brute_force_decode(q, k_pool, v_pool, block_tables, context_lens, scale):
    """Second, independent implementation written with scalar loops."""
    s_count, h_count, d = q.shape
    block_size = k_pool.shape[2]
    out = [[[0.0] * d for _ in range(h_count)] for _ in range(s_count)]
    for s in range(s_count):
        length = int(context_lens[s])
        if length == 0:
            continue
        for h in range(h_count):
            scores = []
            for t in range(length):
                blk = int(block_tables[s][t // block_size])
                off = t % block_size
                dot = math.fsum(float(q[s, h, i]) * float(k_pool[blk, h, off, i])
                                for i in range(d))
                scores.append(float(scale) * dot)
            top = max(scores)
            expo = [math.exp(z - top) for z in scores]
            total = math.fsum(expo)
            for i in range(d):
                acc = []
                for t in range(length):
                    blk = int(block_tables[s][t // block_size])
                    off = t % block_size
                    acc.append(expo[t] * float(v_pool[blk, h, off, i]))
                out[s][h][i] = math.fsum(acc) / total
    return np.array(out, dtype=np.float64)


# ----------------------------------------------------------------------------------
# writes into the pool
# ----------------------------------------------------------------------------------

def cache_append(k_pool, v_pool, key, value, slot_mapping, inplace=False):
    """Pools with row i of key/value written at slot_mapping[i]: copies, or the given
    arrays themselves when ``inplace``.

    key/value [T, H, D]; a negative slot leaves the pools untouched for that row.
    Slots must be distinct."""
    block_size = k_pool.shape[2]
    live = [int(s) for s in slot_mapping if int(s) >= 0]
    if len(set(live)) != len(live):
        raise ValueError("slot_mapping repeats a slot")
    k_out = k_pool if inplace else k_pool.copy()
    v_out = v_pool if inplace else v_pool.copy()
    for i, slot in enumerate(slot_mapping):
        slot = int(slot)
        if slot < 0:
            continue
        b, o = divmod(slot, block_size)
        k_out[b, :, o, :] = key[i]
        v_out[b, :, o, :] = value[i]
    return k_out, v_out


def block_copy(k_pool, v_pool, pairs, inplace=False):
    """Pools with block dst := block src for each (src, dst): copies, or the given
    arrays themselves when ``inplace``.

    All sources are read before any destination is written.  Destinations must be
    distinct and must not be sources."""
    pairs = [(int(a), int(b)) for a, b in np.asarray(pairs).reshape(-1, 2)]
    dsts = [b for _, b in pairs]
    srcs = {a for a, _ in pairs}
    if len(set(dsts)) != len(dsts):
        raise ValueError("block_copy destinations repeat")
    if srcs & set(dsts):
        raise ValueError("block_copy destination is also a source")
    k_src = [k_pool[a].copy() for a, _ in pairs]
    v_src = [v_pool[a].copy() for a, _ in pairs]
    k_out = k_pool if inplace else k_pool.copy()
    v_out = v_pool if inplace else v_pool.copy()
    for (_, b), kb, vb in zip(pairs, k_src, v_src):
        k_out[b] = kb
        v_out[b] = vb
    return k_out, v_out


def swap_blocks(dst_k, dst_v, src_k, src_v, pairs, inplace=False):
    """Destination pools with block dst := source block src for each (src, dst):
    copies, or the given destination arrays themselves when ``inplace``.

    Moving blocks between the GPU pool and host memory under memory pressure and
    back ([Reading vLLM] §3, blocks_to_swap_out / blocks_to_swap_in) copies whole
    blocks, K and V, unchanged.  The two pools may differ in block count.
    Destinations must be distinct."""
    pairs = [(int(a), int(b)) for a, b in np.asarray(pairs).reshape(-1, 2)]
    dsts = [b for _, b in pairs]
    if len(set(dsts)) != len(dsts):
        raise ValueError("swap destinations repeat")
    k_out = dst_k if inplace else dst_k.copy()
    v_out = dst_v if inplace else dst_v.copy()
    for a, b in pairs:
        k_out[b] = src_k[a]
        v_out[b] = src_v[a]
    return k_out, v_out


def slots_for_positions(block_tables, seq_ids, positions, block_size):
    """Slot of (sequence, position) pairs, recomputed from the tables alone."""
    return np.array([slot_of(block_tables[s], p, block_size)
                     for s, p in zip(seq_ids, positions)], dtype=np.int64)
