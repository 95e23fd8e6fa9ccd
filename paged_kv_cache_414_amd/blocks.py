"""Host-side bookkeeping of the paged KV cache: free list, reference counts, block
tables, slot mapping and the copy-on-write trigger.

Pages cited (title, then section):
  [Reading vLLM] "啃透vLLM源码：从PagedAttention到连续批处理，大模型推理加速24倍的秘密"
  [vLLM basics]  "vLLM基础：架构、推理流程与关键组件"

* The cache is cut into fixed-size blocks; a sequence holds only the blocks it needs
  and they may be anywhere in the pool ([Reading vLLM] §2.2; [vLLM basics] §2.3).
* A block table records, per sequence, logical block -> physical block; new blocks
  come from the free list and a finished sequence returns all of its blocks
  ([vLLM basics] §2.3 and the request life cycle of §2.2, steps 4 and 7).
* Physical blocks carry a reference count so that sequences can share them, e.g. a
  common prompt prefix ([Reading vLLM] §2.2, PhysicalTokenBlock.ref_count).
* A sharer that must write into a shared block first gets its own copy
  (copy-on-write, [vLLM basics] §2.3).  Here the first ref_count - 1 writers copy
  and the last remaining holder writes in place.
* Admission follows the scheduler sketch of [Reading vLLM] §3: admit while blocks
  can be allocated, stop at the first request that does not fit.

Slot of logical token ``pos`` of a sequence: table[pos // bs] * bs + pos % bs.
"""

from __future__ import annotations

import dataclasses

import numpy as np


class OutOfBlocks(RuntimeError):
    pass


class BlockAllocator:
    """Physical block ids with reference counts.  A new block is drawn uniformly at
    random from the free list when an RNG is given, else the lowest free id."""

    def __init__(self, num_blocks: int, rng: np.random.Generator | None = None):
        self.num_blocks = int(num_blocks)
        self.ref_count = np.zeros(self.num_blocks, dtype=np.int64)
        self._free = list(range(self.num_blocks))
        if rng is None:
            self._free.reverse()  # pop() then yields the lowest id
        self._rng = rng

    @property
    def num_free(self) -> int:
        return len(self._free)

    def can_allocate(self, n: int) -> bool:
        return n <= len(self._free)

    def allocate(self) -> int:
        if not self._free:
            raise OutOfBlocks("no free block")
        if self._rng is None:
            b = self._free.pop()
        else:
            i = int(self._rng.integers(len(self._free)))
            self._free[i], self._free[-1] = self._free[-1], self._free[i]
            b = self._free.pop()
        self.ref_count[b] = 1
        return b

    def incref(self, b: int) -> None:
        if self.ref_count[b] <= 0:
            raise ValueError(f"block {b} is not allocated")
        self.ref_count[b] += 1

    def decref(self, b: int) -> None:
        if self.ref_count[b] <= 0:
            raise ValueError(f"block {b} is not allocated")
        self.ref_count[b] -= 1
        if self.ref_count[b] == 0:
            self._free.append(int(b))


@dataclasses.dataclass
class Sequence:
    seq_id: int
    blocks: list
    length: int = 0


class BlockManager:
    """Block tables of live sequences over one pool."""

    def __init__(self, num_blocks: int, block_size: int,
                 rng: np.random.Generator | None = None):
        self.block_size = int(block_size)
        self.alloc = BlockAllocator(num_blocks, rng)
        self.seqs: dict[int, Sequence] = {}

    # -- queries ---------------------------------------------------------------------
    def blocks_needed(self, num_tokens: int) -> int:
        return -(-int(num_tokens) // self.block_size)

    def can_allocate(self, num_tokens: int) -> bool:
        return self.alloc.can_allocate(self.blocks_needed(num_tokens))

    def slot(self, seq_id: int, pos: int) -> int:
        seq = self.seqs[seq_id]
        return seq.blocks[pos // self.block_size] * self.block_size + pos % self.block_size

    def context_len(self, seq_id: int) -> int:
        return self.seqs[seq_id].length

    # -- life cycle ----------------------------------------------------------------
    def add_sequence(self, seq_id: int, num_tokens: int) -> np.ndarray:
        """Admit a sequence holding ``num_tokens`` prompt tokens; returns their slots."""
        if seq_id in self.seqs:
            raise ValueError(f"sequence {seq_id} exists")
        n_blk = self.blocks_needed(num_tokens)
        if not self.alloc.can_allocate(n_blk):
            raise OutOfBlocks(f"{n_blk} blocks needed, {self.alloc.num_free} free")
        seq = Sequence(seq_id, [self.alloc.allocate() for _ in range(n_blk)], int(num_tokens))
        self.seqs[seq_id] = seq
        # token p sits in block p // bs at offset p % bs
        per_block = np.asarray(seq.blocks, dtype=np.int64)[:, None] * self.block_size
        slots = (per_block + np.arange(self.block_size)[None, :]).reshape(-1)
        return slots[:num_tokens].astype(np.int32)

    def fork(self, parent_id: int, child_id: int) -> None:
        """The child shares every block of the parent (reference counts + 1)."""
        if child_id in self.seqs:
            raise ValueError(f"sequence {child_id} exists")
        parent = self.seqs[parent_id]
        for b in parent.blocks:
            self.alloc.incref(b)
        self.seqs[child_id] = Sequence(child_id, list(parent.blocks), parent.length)

    def append_slot(self, seq_id: int):
        """Reserve the slot of the sequence's next token.

        Returns (slot, copy) where copy is None or (src, dst): the block that has to be
        duplicated before the token is written, because the sequence shared it."""
        seq = self.seqs[seq_id]
        pos = seq.length
        copy = None
        if pos % self.block_size == 0:
            if pos // self.block_size != len(seq.blocks):
                raise AssertionError("table out of step with length")
            seq.blocks.append(self.alloc.allocate())
        else:
            last = seq.blocks[-1]
            if self.alloc.ref_count[last] > 1:
                new = self.alloc.allocate()
                self.alloc.decref(last)
                seq.blocks[-1] = new
                copy = (int(last), int(new))
        seq.length = pos + 1
        return self.slot(seq_id, pos), copy

    def free(self, seq_id: int) -> None:
        """The sequence finished: every block it holds loses one reference."""
        seq = self.seqs.pop(seq_id)
        for b in seq.blocks:
            self.alloc.decref(b)

    # -- device arrays -------------------------------------------------------------
    def block_tables(self, seq_ids, max_blocks: int, pad: int = 0) -> np.ndarray:
        out = np.full((len(seq_ids), max_blocks), pad, dtype=np.int32)
        for i, sid in enumerate(seq_ids):
            blocks = self.seqs[sid].blocks
            if len(blocks) > max_blocks:
                raise ValueError(f"sequence {sid} holds {len(blocks)} > {max_blocks} blocks")
            out[i, :len(blocks)] = blocks
        return out

    def context_lens(self, seq_ids) -> np.ndarray:
        return np.array([self.seqs[s].length for s in seq_ids], dtype=np.int32)


def slots_for_positions(block_tables: np.ndarray, positions: np.ndarray,
                        block_size: int) -> np.ndarray:
    """slot_mapping for one token per row of ``block_tables`` at ``positions``."""
    rows = np.arange(block_tables.shape[0])
    blk = block_tables[rows, positions // block_size].astype(np.int64)
    return (blk * block_size + positions % block_size).astype(np.int32)


def admit_while_possible(manager: BlockManager, waiting: list) -> list:
    """Admit (seq_id, prompt_len) requests in order while their blocks fit; stop at the
    first that does not ([Reading vLLM] §3, schedule()).  Returns the admitted ids and
    leaves the rest in ``waiting``."""
    admitted = []
    while waiting:
        _, n = waiting[0]
        if not manager.can_allocate(n):
            break
        sid, n = waiting.pop(0)
        manager.add_sequence(sid, n)
        admitted.append(sid)
    return admitted
