"""Step drivers: the host block manager steering the three device entry points.

Each step follows the request life cycle of "vLLM基础：架构、推理流程与关键组件"
(vLLM basics) §2.2: slots for the new tokens are reserved first (a fresh block
when the last one is full, a private copy when the last one is shared), then the
new K/V rows are written, then attention runs with every context length counting
the token just written; finished sequences give their blocks back and new ones are
admitted (continuous batching, same page §2.4).

On the device a step is: pa_block_copy (only when copy-on-write pairs are due),
pa_cache_append of the step's rows, pa_decode, all on the current stream.  After
:meth:`StepMix.prepare`, every step's synthetic inputs (new K/V rows, queries,
prompts of admitted sequences) already sit in HBM, so that a step moves only its
slot mapping, block tables, context lengths and copy pairs from the host (small
copies through torch from pageable memory).

Two step mixes are provided:
  * ContinuousBatching: 64 running sequences; after each step 13 of them finish and
    are replaced by new sequences whose prompt (1-512 tokens) is written by
    pa_cache_append as a stand-in for prefill.
  * SharedPrefix: 8 prompt groups x 8 parallel samples sharing the prompt blocks by
    reference; at the first step each sample's write into the shared, partly filled
    last block triggers copy-on-write ("vLLM basics" §2.3).
"""

from __future__ import annotations

import concurrent.futures
import dataclasses

import numpy as np
import torch

from . import blocks, metrics, ops, workloads


@dataclasses.dataclass
class StepRecord:
    """Everything a step fed to the device, kept on the host for checking."""

    step: int
    copy_pairs: np.ndarray  # int32 [n, 2]
    slots: np.ndarray  # int32 [S], the new token of each batch row
    new_k: np.ndarray
    new_v: np.ndarray
    positions: np.ndarray  # position of each row's new token
    block_tables: np.ndarray
    context_lens: np.ndarray
    q: np.ndarray
    # rows written after the decode (prompts of sequences admitted at this step)
    post_slots: np.ndarray | None = None
    post_k: np.ndarray | None = None
    post_v: np.ndarray | None = None


@dataclasses.dataclass
class StepInputs:
    """One step's random inputs: host arrays, and device copies once staged."""

    new_k: np.ndarray
    new_v: np.ndarray
    q: np.ndarray
    prompt_lens: np.ndarray | None = None  # sequences admitted after the step
    prompt_k: np.ndarray | None = None
    prompt_v: np.ndarray | None = None
    dev: tuple | None = None  # (new_k, new_v, q, prompt_k, prompt_v) on the device


class StepMix:
    """Common driver: subclasses set up sequences and decide who finishes."""

    def __init__(self, spec: workloads.StepMixSpec, draws: workloads.StepDraws,
                 steps: int, max_blocks_per_seq: int, device="cuda",
                 keep_records=False):
        self.spec = spec
        self.draws = draws
        self.steps = int(steps)
        self.mb = int(max_blocks_per_seq)
        self.manager = blocks.BlockManager(spec.num_blocks, spec.block_size,
                                           draws.allocator_rng())
        self.device = device
        torch_dtype = torch.float16 if spec.dtype == np.float16 else torch.float32
        shape = (spec.num_blocks, spec.num_heads, spec.block_size, spec.head_dim)
        self.k_cache = torch.zeros(shape, dtype=torch_dtype, device=device)
        self.v_cache = torch.zeros(shape, dtype=torch_dtype, device=device)
        self.out = torch.empty((spec.num_seqs, spec.num_heads, spec.head_dim),
                               dtype=torch_dtype, device=device)
        self.ws = None
        self.lanes: list[int] = []  # sequence id of each batch row
        self.records: list[StepRecord] = []
        self.keep = keep_records
        self.next_id = 0
        self.initial = None  # (slots, k, v) written before the first step
        self.copies_total = 0
        self.scale = 1.0 / float(np.sqrt(spec.head_dim))
        self.last_decode = None
        self._inputs: dict[int, StepInputs] = {}

    # -- inputs ---------------------------------------------------------------------
    def _draw_inputs(self, k: int) -> StepInputs:
        n = self.spec.num_seqs
        new_k, new_v = self.draws.new_token_kv(k, n)
        return StepInputs(new_k, new_v, self.draws.query(k, n))

    def inputs(self, k: int) -> StepInputs:
        if k not in self._inputs:
            self._inputs[k] = self._draw_inputs(k)
        return self._inputs[k]

    def prepare(self, workers: int = 8) -> None:
        """Draw every step's inputs (on a few threads) and place them in HBM."""
        with concurrent.futures.ThreadPoolExecutor(workers) as pool:
            drawn = list(pool.map(self._draw_inputs, range(self.steps)))
        for k, inp in enumerate(drawn):
            inp.dev = tuple(None if a is None else self.to_dev(a)
                            for a in (inp.new_k, inp.new_v, inp.q, inp.prompt_k, inp.prompt_v))
            self._inputs[k] = inp
        torch.cuda.synchronize()

    # -- helpers ------------------------------------------------------------------
    def to_dev(self, a: np.ndarray) -> torch.Tensor:
        return torch.from_numpy(np.ascontiguousarray(a)).to(self.device)

    def _workspace(self, q, max_ctx):
        need = ops.pa_decode_workspace_bytes(q.shape[0], q.shape[1], q.shape[2],
                                             self.k_cache.shape[2], max_ctx, 0)
        if need and (self.ws is None or self.ws.numel() < need):
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self.ws if need else None

    def _new_id(self) -> int:
        self.next_id += 1
        return self.next_id - 1

    def _append_rows(self, slots, k, v, k_dev=None, v_dev=None):
        if len(slots):
            ops.pa_cache_append(self.k_cache, self.v_cache,
                                self.to_dev(k) if k_dev is None else k_dev,
                                self.to_dev(v) if v_dev is None else v_dev,
                                self.to_dev(slots.astype(np.int32)))

    def _admit_all(self, lens, k_rows, v_rows, k_dev=None, v_dev=None):
        """Admit one sequence per entry of ``lens`` and write their prompt rows."""
        ids, slots = [], []
        for n in lens:
            sid = self._new_id()
            slots.append(self.manager.add_sequence(sid, int(n)))
            ids.append(sid)
        slots = np.concatenate(slots)
        self._append_rows(slots, k_rows, v_rows, k_dev, v_dev)
        return ids, slots

    # -- one step -------------------------------------------------------------------
    def step(self, k_step: int):
        pairs, slots, positions = [], [], []
        for sid in self.lanes:
            pos = self.manager.context_len(sid)
            slot, cow = self.manager.append_slot(sid)
            if cow is not None:
                pairs.append(cow)
            slots.append(slot)
            positions.append(pos)
        pairs = np.array(pairs, dtype=np.int32).reshape(-1, 2)
        slots = np.array(slots, dtype=np.int32)
        tables = self.manager.block_tables(self.lanes, self.mb)
        ctx = self.manager.context_lens(self.lanes)
        max_ctx = int(ctx.max())
        self.copies_total += len(pairs)
        inp = self.inputs(k_step)
        nk_d, nv_d, q_d = inp.dev[:3] if inp.dev else (None, None, None)

        if len(pairs):
            ops.pa_block_copy(self.k_cache, self.v_cache, self.to_dev(pairs))
        self._append_rows(slots, inp.new_k, inp.new_v, nk_d, nv_d)
        q_d = self.to_dev(inp.q) if q_d is None else q_d
        tables_d, ctx_d = self.to_dev(tables), self.to_dev(ctx)
        self.last_decode = self._decode_call(q_d, tables, tables_d, ctx, ctx_d, max_ctx)
        self.last_decode()
        if self.keep:
            self.records.append(StepRecord(k_step, pairs, slots, inp.new_k, inp.new_v,
                                           np.array(positions), tables, ctx, inp.q))
        return ctx

    def _decode_call(self, q_d, tables, tables_d, ctx, ctx_d, max_ctx):
        """The step's decode as a callable (enqueued once per step; again for timing)."""
        ws = self._workspace(q_d, max_ctx)

        def call():
            ops.pa_decode(self.out, q_d, self.k_cache, self.v_cache, tables_d, ctx_d,
                          self.scale, max_ctx, 0, ws)
        return call

    def decode_again(self):
        """Enqueue the last step's decode once more (same inputs; for timing)."""
        self.last_decode()

    def kv_bytes(self, ctx) -> int:
        return metrics.decode_kv_bytes(ctx, self.spec.num_heads, self.spec.head_dim,
                                       np.dtype(self.spec.dtype).itemsize)


class ContinuousBatching(StepMix):
    """64 running sequences, 13 replaced after every step (see module docstring)."""

    def __init__(self, seed: int, steps: int | None = None, device="cuda",
                 keep_records=False):
        spec = workloads.CONTINUOUS_BATCHING
        draws = workloads.ContinuousBatchingDraws(spec, seed)
        steps = steps or spec.steps
        mb = -(-(draws.prompt_high + steps) // spec.block_size)
        super().__init__(spec, draws, steps, mb, device, keep_records)
        lens = draws.initial_prompt_lens()
        k, v = draws.prompt_kv(-1, lens)
        self.lanes, slots = self._admit_all(lens, k, v)
        self.initial = (slots, k, v)

    def _draw_inputs(self, k: int) -> StepInputs:
        inp = super()._draw_inputs(k)
        inp.prompt_lens = self.draws.replacement_prompt_lens(k)
        inp.prompt_k, inp.prompt_v = self.draws.prompt_kv(k, inp.prompt_lens)
        return inp

    def run_step(self, k_step: int):
        ctx = self.step(k_step)
        # retire and admit; the new prompts are written before the next step
        inp = self.inputs(k_step)
        finishing = self.draws.finishing(k_step)
        for lane in finishing:
            self.manager.free(self.lanes[lane])
        k_dev, v_dev = inp.dev[3:] if inp.dev else (None, None)
        ids, slots = self._admit_all(inp.prompt_lens, inp.prompt_k, inp.prompt_v, k_dev, v_dev)
        for lane, sid in zip(finishing, ids):
            self.lanes[lane] = sid
        if self.keep:
            rec = self.records[-1]
            rec.post_slots, rec.post_k, rec.post_v = slots, inp.prompt_k, inp.prompt_v
        return ctx


class SharedPrefix(StepMix):
    """8 groups x 8 samples sharing their prompt blocks (see module docstring).

    With ``shared_decode`` the decode runs through pa_decode_shared_prefix: each
    group's leading blocks that all of its samples still hold are read once for the
    whole group."""

    def __init__(self, seed: int, steps: int | None = None, device="cuda",
                 keep_records=False, shared_decode=False):
        self.shared_decode = bool(shared_decode)
        self.ws_shared = None
        spec = workloads.SHARED_PREFIX
        draws = workloads.SharedPrefixDraws(spec, seed)
        steps = steps or spec.steps
        lens = draws.prompt_lens()
        mb = -(-(int(lens.max()) + steps) // spec.block_size)
        super().__init__(spec, draws, steps, mb, device, keep_records)
        k, v = draws.prompt_kv(-1, lens)
        leaders, slots = self._admit_all(lens, k, v)
        for leader in leaders:
            group = [leader]
            for _ in range(draws.samples - 1):
                child = self._new_id()
                self.manager.fork(leader, child)
                group.append(child)
            self.lanes.extend(group)
        self.initial = (slots, k, v)

    def shared_prefix(self, tables: np.ndarray, ctx: np.ndarray):
        """(group_starts, prefix_lens): the lanes of a group are contiguous; its
        prefix is the leading whole blocks whose ids every member's table holds."""
        n = self.draws.samples
        starts = np.arange(0, len(self.lanes) + 1, n, dtype=np.int32)
        prefix = np.zeros(len(self.lanes), dtype=np.int32)
        bs = self.spec.block_size
        for r0 in starts[:-1]:
            rows = tables[r0:r0 + n]
            same = np.all(rows == rows[0], axis=0)
            lead = int(np.argmin(same)) if not same.all() else same.size
            lead = min(lead, int(ctx[r0:r0 + n].min()) // bs)
            prefix[r0:r0 + n] = lead * bs
        return starts, prefix

    def _decode_call(self, q_d, tables, tables_d, ctx, ctx_d, max_ctx):
        if not self.shared_decode:
            return super()._decode_call(q_d, tables, tables_d, ctx, ctx_d, max_ctx)
        starts, prefix = self.shared_prefix(tables, ctx)
        max_prefix = int(prefix.max())
        max_suffix = int((ctx - prefix).max())
        starts_d, prefix_d = self.to_dev(starts), self.to_dev(prefix)
        need = ops.pa_decode_shared_prefix_workspace_bytes(
            q_d.shape[0], q_d.shape[1], q_d.shape[2], self.spec.block_size, len(starts) - 1,
            max_prefix, max_suffix)
        if self.ws_shared is None or self.ws_shared.numel() < need:
            self.ws_shared = torch.empty(need, dtype=torch.uint8, device=self.device)
        ws = self.ws_shared

        def call():
            ops.pa_decode_shared_prefix(self.out, q_d, self.k_cache, self.v_cache, tables_d,
                                        ctx_d, starts_d, prefix_d, self.scale, max_prefix,
                                        max_suffix, workspace=ws)
        return call

    def run_step(self, k_step: int):
        return self.step(k_step)
