"""Seeded synthetic inputs for the paged decode path.

This module only draws random numbers and lays them out; it performs none of the
attention, append or copy arithmetic.  Both the HIP path and the CPU oracle take
their inputs from here.

Workload shapes follow what the pages describe:
  * blocks of 16 tokens by default, scattered anywhere in a physical pool and reached
    through a per-sequence table of physical block ids ("Reading the vLLM source ..."
    §2.2; "vLLM basics: architecture, inference flow and key components" §2.3);
  * 96 concurrent sequences, 32 heads of dimension 128, contexts between the average
    of 300 and the maximum of 2048 tokens ("Reading the vLLM source ..." §1 table;
    "vLLM basics ..." §2.3 and the §2.5 case study);
  * parallel samples sharing prompt blocks ("vLLM basics ..." §2.3, copy-on-write);
  * a 32-token block size for long text ("Reading the vLLM source ..." §2.3).

Values are N(0, 1) drawn in float32 by numpy's PCG64 and, for half precision,
rounded to nearest even.  The draw order is fixed: context lengths, then block ids,
then q, then K, then V.

Unused pool memory can be filled with NaN ("poisoned") so that a kernel reading
anything outside the live tokens shows up in the output.  Table entries past a
sequence's last live block are filled with the id of a poisoned block (always a
valid index, never an out-of-range one).
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os

import numpy as np

F16_NAN_BITS = np.uint16(0x7E00)
F32_NAN_BITS = np.uint32(0x7FC00000)

# Elements per independently drawn chunk of a large array (bounds temporary memory).
_FILL_CHUNK = 1 << 22


@dataclasses.dataclass
class DecodeBatch:
    """One decode call's inputs, all host numpy arrays."""

    name: str
    dtype: np.dtype
    num_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    q: np.ndarray  # [S, H, D]
    k_pool: np.ndarray  # [NB, H, bs, D]
    v_pool: np.ndarray  # [NB, H, bs, D]
    block_tables: np.ndarray  # int32 [S, MB]
    context_lens: np.ndarray  # int32 [S]
    scale: float

    @property
    def num_seqs(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0


# ----------------------------------------------------------------------------------
# random fills
# ----------------------------------------------------------------------------------

def fill_normal(rng: np.random.Generator, out: np.ndarray) -> None:
    """Fill ``out`` (float16 or float32, C-contiguous) with N(0,1) drawn in float32.

    The array is cut into fixed chunks of _FILL_CHUNK elements; chunk i is drawn from
    the i-th child generator spawned from ``rng``, on a few threads for large arrays.
    The values depend neither on the number of threads nor, for a given leading
    part of the array, on the array's total size."""
    flat = out.reshape(-1)
    starts = list(range(0, flat.size, _FILL_CHUNK))
    if not starts:
        return
    children = rng.spawn(len(starts))

    def fill(i):
        start = starts[i]
        stop = min(flat.size, start + _FILL_CHUNK)
        vals = children[i].standard_normal(stop - start, dtype=np.float32)
        flat[start:stop] = vals  # float16 destination: numpy rounds to nearest even

    workers = max(1, min(16, os.cpu_count() or 1, len(starts)))
    if workers == 1:
        fill(0)
        return
    with concurrent.futures.ThreadPoolExecutor(workers) as pool:
        list(pool.map(fill, range(len(starts))))


def normal(rng: np.random.Generator, shape, dtype) -> np.ndarray:
    out = np.empty(shape, dtype=dtype)
    fill_normal(rng, out)
    return out


def nan_bits_for(dtype) -> tuple[np.dtype, int]:
    dtype = np.dtype(dtype)
    if dtype == np.float16:
        return np.dtype(np.uint16), int(F16_NAN_BITS)
    if dtype == np.float32:
        return np.dtype(np.uint32), int(F32_NAN_BITS)
    raise ValueError(f"unsupported dtype {dtype}")


def poison_pool(pool: np.ndarray, live_mask: np.ndarray) -> None:
    """Write NaN into every token slot of ``pool`` [NB, H, bs, D] where
    ``live_mask`` [NB, bs] is False."""
    itype, bits = nan_bits_for(pool.dtype)
    view = pool.view(itype)
    blocks, offs = np.nonzero(~live_mask)
    # pool[b, :, o, :] for every dead (b, o)
    view[blocks, :, offs, :] = bits


# ----------------------------------------------------------------------------------
# static decode batches
# ----------------------------------------------------------------------------------

def _deal_tables(ctx: np.ndarray, block_size: int, ids: np.ndarray, max_blocks: int,
                 pad_id: int) -> np.ndarray:
    """Hand out ``ids`` in order: sequence 0 takes the first ceil(ctx0/bs), and so on."""
    tables = np.full((ctx.size, max_blocks), pad_id, dtype=np.int32)
    cursor = 0
    for s, n_tok in enumerate(ctx):
        n_blk = -(-int(n_tok) // block_size)
        tables[s, :n_blk] = ids[cursor:cursor + n_blk]
        cursor += n_blk
    return tables


def _live_mask(tables: np.ndarray, ctx: np.ndarray, block_size: int,
               num_blocks: int) -> np.ndarray:
    live = np.zeros((num_blocks, block_size), dtype=bool)
    for s, n_tok in enumerate(ctx):
        n_tok = int(n_tok)
        n_blk = -(-n_tok // block_size)
        for j in range(n_blk):
            take = min(block_size, n_tok - j * block_size)
            live[tables[s, j], :take] = True
    return live


def make_static_batch(name: str, *, seed: int, num_seqs: int, num_heads: int,
                      head_dim: int, block_size: int, ctx_low: int, ctx_high: int,
                      dtype, num_blocks: int | None = None, pool_slack: float = 1.1,
                      max_blocks_per_seq: int | None = None, scale: float | None = None,
                      poison: bool = True) -> DecodeBatch:
    """Draw a decode batch: context lengths uniform in [ctx_low, ctx_high], block ids
    a seeded random permutation of the pool dealt out in order, q/K/V ~ N(0,1)."""
    dtype = np.dtype(dtype)
    rng = np.random.default_rng(seed)
    ctx = rng.integers(ctx_low, ctx_high + 1, size=num_seqs).astype(np.int32)
    needed = int(sum(-(-int(c) // block_size) for c in ctx))
    if num_blocks is None:  # at least one block, for the table padding of empty contexts
        num_blocks = max(1, int(math.ceil(pool_slack * needed)))
    if needed > num_blocks:
        raise ValueError(f"{name}: {needed} blocks needed, pool has {num_blocks}")
    if max_blocks_per_seq is None:
        max_blocks_per_seq = -(-ctx_high // block_size)
    perm = rng.permutation(num_blocks).astype(np.int32)
    # entries past a sequence's last live block point at an unused (poisoned) block
    pad_id = int(perm[needed]) if needed < num_blocks else int(perm[0])
    tables = _deal_tables(ctx, block_size, perm, max_blocks_per_seq, pad_id)
    q = normal(rng, (num_seqs, num_heads, head_dim), dtype)
    k_pool = normal(rng, (num_blocks, num_heads, block_size, head_dim), dtype)
    v_pool = normal(rng, (num_blocks, num_heads, block_size, head_dim), dtype)
    if poison:
        live = _live_mask(tables, ctx, block_size, num_blocks)
        poison_pool(k_pool, live)
        poison_pool(v_pool, live)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return DecodeBatch(name=name, dtype=dtype, num_heads=num_heads, head_dim=head_dim,
                       block_size=block_size, num_blocks=num_blocks,
                       max_blocks_per_seq=max_blocks_per_seq, q=q, k_pool=k_pool,
                       v_pool=v_pool, block_tables=tables, context_lens=ctx,
                       scale=float(scale))


def tiny_fp32(seed: int = 1, poison: bool = True) -> DecodeBatch:
    """4 seqs x 4 heads x 64, block 16, pool of 64 blocks, contexts U[1, 64], fp32."""
    return make_static_batch("tiny_fp32", seed=seed, num_seqs=4, num_heads=4,
                             head_dim=64, block_size=16, ctx_low=1, ctx_high=64,
                             dtype=np.float32, num_blocks=64, max_blocks_per_seq=4,
                             scale=1.0 / 8.0, poison=poison)


def llama7b_decode(seed: int = 2, poison: bool = True, num_seqs: int = 96) -> DecodeBatch:
    """Llama-7B-shaped layer: 96 seqs x 32 heads x 128, block 16, contexts
    U[300, 2048], pool sized to 110% of the blocks needed, fp16."""
    return make_static_batch("llama7b_decode", seed=seed, num_seqs=num_seqs,
                             num_heads=32, head_dim=128, block_size=16, ctx_low=300,
                             ctx_high=2048, dtype=np.float16, pool_slack=1.1,
                             poison=poison)


def long_context(seed: int = 5, poison: bool = True, num_seqs: int = 8) -> DecodeBatch:
    """8 seqs x 32 heads x 128, block 32, contexts U[16384, 32768], a pool of
    10,000 blocks, fp16."""
    return make_static_batch("long_context", seed=seed, num_seqs=num_seqs, num_heads=32,
                             head_dim=128, block_size=32, ctx_low=16384,
                             ctx_high=32768, dtype=np.float16, num_blocks=10_000,
                             poison=poison)


@dataclasses.dataclass
class SharedPrefixBatch(DecodeBatch):
    """A decode batch whose sequences come in groups sharing their leading blocks.

    Group g is sequences [group_starts[g], group_starts[g + 1]); each of them shares
    its first prefix_lens[s] tokens (whole blocks, the same physical ids) with the
    rest of its group.  Sequences outside every group have prefix_lens 0."""

    group_starts: np.ndarray = None  # int32 [G + 1]
    prefix_lens: np.ndarray = None  # int32 [S]

    @property
    def num_groups(self) -> int:
        return int(self.group_starts.size - 1)

    @property
    def max_prefix_len(self) -> int:
        return int(self.prefix_lens.max()) if self.prefix_lens.size else 0

    @property
    def max_suffix_len(self) -> int:
        if not self.context_lens.size:
            return 0
        return int((self.context_lens - self.prefix_lens).max())


def make_shared_prefix_batch(name: str, *, seed: int, group_sizes, num_heads: int,
                             head_dim: int, block_size: int, prefix_blocks_low: int,
                             prefix_blocks_high: int, suffix_low: int, suffix_high: int,
                             ungrouped: int = 0, dtype=np.float16, pool_slack: float = 1.1,
                             scale: float | None = None,
                             poison: bool = True) -> SharedPrefixBatch:
    """Draw a grouped batch: ``ungrouped`` unshared sequences first, then one group per
    entry of ``group_sizes``.  A group's prefix is U[prefix_blocks_low,
    prefix_blocks_high] whole blocks, each sequence's own tokens after it are
    U[suffix_low, suffix_high] (ungrouped sequences: that many tokens in all).  Block
    ids are a seeded random permutation of the pool, dealt out in order: a group's
    shared blocks once, then every member's own blocks."""
    dtype = np.dtype(dtype)
    rng = np.random.default_rng(seed)
    group_sizes = [int(n) for n in group_sizes]
    prefix_blocks = rng.integers(prefix_blocks_low, prefix_blocks_high + 1,
                                 size=len(group_sizes)).astype(np.int64)
    num_seqs = int(ungrouped) + sum(group_sizes)
    suffix = rng.integers(suffix_low, suffix_high + 1, size=num_seqs).astype(np.int64)
    prefix_lens = np.zeros(num_seqs, dtype=np.int64)
    starts = [int(ungrouped)]
    for g, n in enumerate(group_sizes):
        prefix_lens[starts[-1]:starts[-1] + n] = prefix_blocks[g] * block_size
        starts.append(starts[-1] + n)
    ctx = (prefix_lens + suffix).astype(np.int32)
    own_blocks = [-(-int(c) // block_size) - int(p) // block_size
                  for c, p in zip(ctx, prefix_lens)]
    needed = int(prefix_blocks.sum()) + sum(own_blocks)
    num_blocks = max(int(math.ceil(pool_slack * needed)), needed + 1)
    max_blocks = max(1, max(-(-int(c) // block_size) for c in ctx) if num_seqs else 1)
    perm = rng.permutation(num_blocks).astype(np.int32)
    pad_id = int(perm[needed])  # an unused block: poisoned, never live
    tables = np.full((num_seqs, max_blocks), pad_id, dtype=np.int32)
    cursor = 0
    for s in range(int(ungrouped)):
        tables[s, :own_blocks[s]] = perm[cursor:cursor + own_blocks[s]]
        cursor += own_blocks[s]
    for g, n in enumerate(group_sizes):
        shared = perm[cursor:cursor + int(prefix_blocks[g])]
        cursor += int(prefix_blocks[g])
        for s in range(starts[g], starts[g + 1]):
            tables[s, :shared.size] = shared
            tables[s, shared.size:shared.size + own_blocks[s]] = perm[cursor:cursor + own_blocks[s]]
            cursor += own_blocks[s]
    q = normal(rng, (num_seqs, num_heads, head_dim), dtype)
    k_pool = normal(rng, (num_blocks, num_heads, block_size, head_dim), dtype)
    v_pool = normal(rng, (num_blocks, num_heads, block_size, head_dim), dtype)
    if poison:
        live = _live_mask(tables, ctx, block_size, num_blocks)
        poison_pool(k_pool, live)
        poison_pool(v_pool, live)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return SharedPrefixBatch(name=name, dtype=dtype, num_heads=num_heads, head_dim=head_dim,
                             block_size=block_size, num_blocks=num_blocks,
                             max_blocks_per_seq=max_blocks, q=q, k_pool=k_pool,
                             v_pool=v_pool, block_tables=tables, context_lens=ctx,
                             scale=float(scale),
                             group_starts=np.asarray(starts, dtype=np.int32),
                             prefix_lens=prefix_lens.astype(np.int32))


def shared_prefix_decode(seed: int = 4, poison: bool = True) -> SharedPrefixBatch:
    """The shared-prefix mix at its last step as one batch: 8 groups x 8 samples x 32
    heads x 128, block 16, fp16; every group shares a 1024-token prefix (64 blocks)
    and each sample holds 257-271 tokens of its own (1-15 prompt tokens past the
    prefix plus 256 generated ones)."""
    return make_shared_prefix_batch("shared_prefix_decode", seed=seed, group_sizes=[8] * 8,
                                    num_heads=32, head_dim=128, block_size=16,
                                    prefix_blocks_low=64, prefix_blocks_high=64,
                                    suffix_low=257, suffix_high=271, poison=poison)


# ----------------------------------------------------------------------------------
# dynamic step mixes: random decisions and values only; block bookkeeping is done
# by the host allocator
# ----------------------------------------------------------------------------------

@dataclasses.dataclass
class StepMixSpec:
    name: str
    num_seqs: int
    num_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    steps: int
    dtype: np.dtype


CONTINUOUS_BATCHING = StepMixSpec("continuous_batching", num_seqs=64, num_heads=32,
                                  head_dim=128, block_size=16, num_blocks=2560,
                                  steps=50, dtype=np.dtype(np.float16))
SHARED_PREFIX = StepMixSpec("shared_prefix_cow", num_seqs=64, num_heads=32,
                            head_dim=128, block_size=16, num_blocks=2048, steps=256,
                            dtype=np.dtype(np.float16))


class StepDraws:
    """Per-step random draws for a step mix, reproducible step by step.

    Each step has its own generator seeded by (seed, step), so a test that runs only
    the first few steps sees the same values as a run of all of them."""

    def __init__(self, spec: StepMixSpec, seed: int):
        self.spec = spec
        self.seed = int(seed)

    def rng(self, step: int, stream: int = 0) -> np.random.Generator:
        # step -1 stands for draws made before the first step
        return np.random.default_rng([self.seed, int(step) + 1, int(stream)])

    def allocator_seed(self) -> int:
        """Non-zero seed of the block manager's random choice of free blocks."""
        return int(np.random.default_rng([self.seed, 1 << 20]).integers(1, 1 << 62))

    def new_token_kv(self, step: int, n: int) -> tuple[np.ndarray, np.ndarray]:
        s = self.spec
        rng = self.rng(step, 1)
        k = normal(rng, (n, s.num_heads, s.head_dim), s.dtype)
        v = normal(rng, (n, s.num_heads, s.head_dim), s.dtype)
        return k, v

    def query(self, step: int, n: int) -> np.ndarray:
        s = self.spec
        return normal(self.rng(step, 2), (n, s.num_heads, s.head_dim), s.dtype)

    def prompt_kv(self, step: int, lens) -> tuple[np.ndarray, np.ndarray]:
        """K and V rows of the prompts admitted at ``step`` (step -1: before the first
        step), concatenated in admission order: [sum(lens), H, D] each."""
        s = self.spec
        rng = self.rng(step, 4)
        n = int(np.sum(lens))
        k = normal(rng, (n, s.num_heads, s.head_dim), s.dtype)
        v = normal(rng, (n, s.num_heads, s.head_dim), s.dtype)
        return k, v


class ContinuousBatchingDraws(StepDraws):
    """64 running sequences; after each step 20% of them (13) finish and are replaced by
    new ones whose prompt length is uniform in [1, 512]."""

    finish_fraction = 0.2
    prompt_low = 1
    prompt_high = 512

    @property
    def finish_count(self) -> int:
        return int(round(self.finish_fraction * self.spec.num_seqs))

    def initial_prompt_lens(self) -> np.ndarray:
        rng = self.rng(-1, 3)
        return rng.integers(self.prompt_low, self.prompt_high + 1,
                            size=self.spec.num_seqs).astype(np.int32)

    def finishing(self, step: int) -> np.ndarray:
        rng = self.rng(step, 3)
        return np.sort(rng.choice(self.spec.num_seqs, size=self.finish_count,
                                  replace=False)).astype(np.int32)

    def replacement_prompt_lens(self, step: int) -> np.ndarray:
        rng = self.rng(step, 6)
        return rng.integers(self.prompt_low, self.prompt_high + 1,
                            size=self.finish_count).astype(np.int32)


class SharedPrefixDraws(StepDraws):
    """8 prompt groups x 8 parallel samples.  Each group's prompt is 1024 tokens (64
    full blocks) plus 1-15 extra tokens that share a 65th, partly filled block, so
    that the first divergent write of each sample lands in a shared block."""

    groups = 8
    samples = 8
    prefix_tokens = 1024
    extra_low = 1
    extra_high = 15

    def prompt_lens(self) -> np.ndarray:
        rng = self.rng(-1, 5)
        extra = rng.integers(self.extra_low, self.extra_high + 1, size=self.groups)
        return (self.prefix_tokens + extra).astype(np.int32)
