"""Host-side bookkeeping of the paged KV cache: the native block manager of
``libpa.so`` (include/pa_blocks.h) under a small Python class, plus two helpers.

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
  (copy-on-write, [vLLM basics] §2.3).  The first ref_count - 1 writers copy and the
  last remaining holder writes in place.
* Admission follows the scheduler sketch of [Reading vLLM] §3: admit while blocks
  can be allocated, stop at the first request that does not fit.

Slot of logical token ``pos`` of a sequence: table[pos // bs] * bs + pos % bs.
"""

from __future__ import annotations

import numpy as np

from . import ops


class OutOfBlocks(RuntimeError):
    pass


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _ids(seq_ids) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64).reshape(-1))


class BlockManager:
    """Block tables of live sequences over one pool of ``num_blocks`` blocks.

    seed None or 0: a new block is the most recently freed one (initially the lowest
    id); otherwise new blocks are drawn uniformly from the free list (SplitMix64
    seeded with ``seed``)."""

    def __init__(self, num_blocks: int, block_size: int, seed: int | None = None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self._lib = ops.lib
        self._h = self._lib.pa_bm_create(self.num_blocks, self.block_size, int(seed or 0))
        if not self._h:
            raise ValueError(self._lib.pa_last_error().decode())

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            self._lib.pa_bm_destroy(h)

    def _check(self, status: int) -> None:
        if status == 0:
            return
        msg = self._lib.pa_last_error().decode()
        if status == 6:
            raise OutOfBlocks(msg)
        if status == 2:
            raise ValueError(msg)
        raise ops.PagedAttentionError(status, msg)

    # -- queries ---------------------------------------------------------------------
    @property
    def num_free(self) -> int:
        return int(self._lib.pa_bm_num_free(self._h))

    def blocks_needed(self, num_tokens: int) -> int:
        return -(-int(num_tokens) // self.block_size)

    def can_allocate(self, num_tokens: int) -> bool:
        return bool(self._lib.pa_bm_can_allocate(self._h, int(num_tokens)))

    def ref_counts(self) -> np.ndarray:
        out = np.empty(self.num_blocks, dtype=np.int32)
        self._check(self._lib.pa_bm_ref_counts(self._h, _ptr(out)))
        return out

    def blocks_of(self, seq_id: int) -> list:
        n = int(self._lib.pa_bm_num_seq_blocks(self._h, int(seq_id)))
        if n < 0:
            raise ValueError(f"unknown sequence {seq_id}")
        out = np.empty(max(n, 1), dtype=np.int32)
        self._check(self._lib.pa_bm_seq_blocks(self._h, int(seq_id), _ptr(out), n))
        return out[:n].tolist()

    def context_len(self, seq_id: int) -> int:
        return int(self.context_lens([seq_id])[0])

    def slot(self, seq_id: int, pos: int) -> int:
        blocks = self.blocks_of(seq_id)
        return blocks[pos // self.block_size] * self.block_size + pos % self.block_size

    # -- life cycle ----------------------------------------------------------------
    def add_sequence(self, seq_id: int, num_tokens: int, slots: np.ndarray | None = None) -> np.ndarray:
        """Admit a sequence holding ``num_tokens`` prompt tokens; returns their slots
        (written into ``slots`` when given, an int32 array of at least that length)."""
        n = int(num_tokens)
        out = np.empty(max(n, 1), dtype=np.int32) if slots is None else slots
        self._check(self._lib.pa_bm_add_sequence(self._h, int(seq_id), n, _ptr(out)))
        return out[:n]

    def add_sequences(self, seq_ids, num_tokens, slots: np.ndarray | None = None) -> np.ndarray:
        """Admit several sequences at once (all or nothing); returns their prompt
        tokens' slots, concatenated in order (written into ``slots`` when given)."""
        ids = _ids(seq_ids)
        lens = np.ascontiguousarray(np.asarray(num_tokens, dtype=np.int32).reshape(-1))
        total = int(lens.sum())
        out = np.empty(max(total, 1), dtype=np.int32) if slots is None else slots
        self._check(self._lib.pa_bm_add_sequences(self._h, _ptr(ids), _ptr(lens), ids.size,
                                                  _ptr(out)))
        return out[:total]

    def fork(self, parent_id: int, child_id: int) -> None:
        """The child shares every block of the parent (reference counts + 1)."""
        self._check(self._lib.pa_bm_fork(self._h, int(parent_id), int(child_id)))

    def free(self, seq_id: int) -> None:
        """The sequence finished: every block it holds loses one reference."""
        self._check(self._lib.pa_bm_free(self._h, int(seq_id)))

    def append_slots(self, seq_ids, slots=None, positions=None, pairs=None):
        """Reserve the next token's slot of each listed sequence (all or nothing).

        Returns (slots int32 [n], positions int32 [n], copy pairs int32 [c, 2]); the
        pairs are blocks to duplicate (source, destination) before the tokens are
        written.  Output arrays may be passed in (e.g. views of a staging buffer)."""
        ids = _ids(seq_ids)
        n = ids.size
        slots = np.empty(max(n, 1), dtype=np.int32) if slots is None else slots
        positions = np.empty(max(n, 1), dtype=np.int32) if positions is None else positions
        pairs = np.empty((max(n, 1), 2), dtype=np.int32) if pairs is None else pairs
        count = np.zeros(1, dtype=np.int32)
        self._check(self._lib.pa_bm_append_slots(self._h, _ptr(ids), n, _ptr(slots),
                                                 _ptr(positions), _ptr(pairs), _ptr(count)))
        return slots[:n], positions[:n], pairs[:int(count[0])]

    def append_slot(self, seq_id: int):
        """(slot, copy) for one sequence; copy is None or (src, dst)."""
        slots, _, pairs = self.append_slots([seq_id])
        copy = (int(pairs[0, 0]), int(pairs[0, 1])) if len(pairs) else None
        return int(slots[0]), copy

    # -- device arrays -------------------------------------------------------------
    def block_tables(self, seq_ids, max_blocks: int, pad: int = 0,
                     out: np.ndarray | None = None) -> np.ndarray:
        ids = _ids(seq_ids)
        out = np.empty((ids.size, int(max_blocks)), dtype=np.int32) if out is None else out
        self._check(self._lib.pa_bm_block_tables(self._h, _ptr(ids), ids.size, int(max_blocks),
                                                 int(pad), _ptr(out)))
        return out

    def context_lens(self, seq_ids, out: np.ndarray | None = None) -> np.ndarray:
        ids = _ids(seq_ids)
        out = np.empty(max(ids.size, 1), dtype=np.int32) if out is None else out
        self._check(self._lib.pa_bm_context_lens(self._h, _ptr(ids), ids.size, _ptr(out)))
        return out[:ids.size]

    def shared_prefix_blocks(self, seq_ids) -> int:
        """Leading whole blocks that every listed sequence holds as the same physical
        blocks."""
        ids = _ids(seq_ids)
        n = int(self._lib.pa_bm_shared_prefix_blocks(self._h, _ptr(ids), ids.size))
        if n < 0:
            raise ValueError(self._lib.pa_last_error().decode())
        return n


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
