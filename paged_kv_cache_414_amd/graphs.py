"""A decode step captured once as a HIP graph and replayed.

"Reading the vLLM source ..." §4 captures the model step in a graph after warm-up
runs and replays it, to save launch overhead at small batch.  The step here is the
path's own: pa_cache_append of each sequence's newest K/V row, then pa_decode.

Both entry points only validate arguments on the host and enqueue kernels -- no
allocation, no synchronisation, no memset -- so they can be recorded into a graph
as they are.  A graph replays with the pointers and sizes it was recorded with, so
the step works on fixed device buffers: the caller writes each step's queries, new
rows, slots, block tables and context lengths into them (e.g. one copy from a
staging buffer) and replays.  Two sizes must be fixed at capture: the number of
sequences (rows of a smaller batch can be retired by a context length of 0 and a
slot of -1) and an upper bound of the context length, which sizes the decode grid;
partitions past a sequence's context end at once.

With ``fused=True`` the step is the single launch of pa_decode_append: each row's new
K/V goes to position context_lens[s] - 1 (a retired row, context 0, writes nothing)
and ``slots`` is not used.
"""

from __future__ import annotations

import torch

from . import ops


class DecodeStepGraph:
    """pa_cache_append + pa_decode over fixed buffers, recorded once, replayed per step.

    Buffers (write them before :meth:`replay`): ``q``, ``new_k``, ``new_v``
    [S, H, D]; ``slots`` int32 [S]; ``block_tables`` int32 [S, MB]; ``context_lens``
    int32 [S] (each <= ``max_context_len``).  Result: ``out`` [S, H, D]."""

    def __init__(self, key_cache: torch.Tensor, value_cache: torch.Tensor, num_seqs: int,
                 max_blocks_per_seq: int, max_context_len: int, scale: float,
                 partition_size: int = 0, fused: bool = False):
        nb, h, bs, d = key_cache.shape
        dev = key_cache.device
        self.k_cache, self.v_cache = key_cache, value_cache
        self.scale = float(scale)
        self.max_context_len = int(max_context_len)
        self.partition_size = int(partition_size)
        self.fused = bool(fused)
        s = int(num_seqs)
        self.q = torch.zeros((s, h, d), dtype=key_cache.dtype, device=dev)
        self.new_k = torch.zeros_like(self.q)
        self.new_v = torch.zeros_like(self.q)
        self.out = torch.zeros_like(self.q)
        self.slots = torch.full((s,), -1, dtype=torch.int32, device=dev)
        self.block_tables = torch.zeros((s, int(max_blocks_per_seq)), dtype=torch.int32, device=dev)
        self.context_lens = torch.zeros((s,), dtype=torch.int32, device=dev)
        self.workspace = ops.workspace_for(self.q, key_cache, self.max_context_len,
                                           self.partition_size)
        # warm-up outside the graph (kernel code objects are loaded on first launch),
        # on a side stream as graph capture requires; slots of -1 and empty contexts
        # make these launches touch nothing
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            for _ in range(2):
                self._enqueue()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize(dev)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self._enqueue()

    def _enqueue(self) -> None:
        if self.fused:
            ops.pa_decode_append(self.out, self.q, self.k_cache, self.v_cache, self.new_k,
                                 self.new_v, self.block_tables, self.context_lens, self.scale,
                                 self.max_context_len, self.partition_size, self.workspace)
            return
        ops.pa_cache_append(self.k_cache, self.v_cache, self.new_k, self.new_v, self.slots)
        ops.pa_decode(self.out, self.q, self.k_cache, self.v_cache, self.block_tables,
                      self.context_lens, self.scale, self.max_context_len,
                      self.partition_size, self.workspace)

    def run_eager(self) -> None:
        """The same step launched directly (for comparison)."""
        self._enqueue()

    def replay(self) -> None:
        self.graph.replay()
