"""Step drivers: the host block manager steering the device entry points.

Each step follows the request life cycle of "vLLM基础：架构、推理流程与关键组件"
(vLLM basics) §2.2: slots for the new tokens are reserved first (a fresh block
when the last one is full, a private copy when the last one is shared), then the
new K/V rows are written, then attention runs with every context length counting
the token just written; finished sequences give their blocks back and new ones are
admitted (continuous batching, same page §2.4).

Host side of a step (native block manager, include/pa_blocks.h): reserve the slots
of every running sequence, build the block tables and context lengths, and for a
continuous-batching step retire the finished sequences and admit new ones.  Every
small array the device needs is written straight into one pinned staging buffer
(two, used in turn) and moved with one asynchronous copy.  Device side, all on the
current stream: pa_block_copy (only when copy-on-write pairs are due),
pa_cache_append of the step's rows, the decode (pa_decode, or
pa_decode_shared_prefix), then pa_cache_append of admitted prompts.  With
``native=True`` the whole step is one call of the decode-step executor
(include/pa_step.h, :mod:`engine`), which does the same in the same order.  After
:meth:`StepMix.prepare`, every step's synthetic inputs (new K/V rows, queries,
prompts) already sit in HBM.

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
    finishing: np.ndarray | None = None  # batch rows that finish after the step
    prompt_k: np.ndarray | None = None
    prompt_v: np.ndarray | None = None
    dev: tuple | None = None  # (new_k, new_v, q, prompt_k, prompt_v) on the device


class Staging:
    """Small int32 arrays of one step, written on the host into a pinned buffer and
    moved to the device with one asynchronous copy.  Two pinned buffers are used in
    turn; before one is rewritten, the copy that last read it has completed.  The
    device buffer is reused every step: stream order puts the next copy after every
    kernel that reads the previous step's arrays."""

    ALIGN = 4  # int32 elements (16 bytes)

    def __init__(self, capacity: int, device):
        self.capacity = int(capacity)
        self.host = [torch.empty(self.capacity, dtype=torch.int32, pin_memory=True)
                     for _ in range(2)]
        self.host_np = [h.numpy() for h in self.host]
        self.events = [None, None]
        self.dev = torch.empty(self.capacity, dtype=torch.int32, device=device)
        self.turn = 0
        self.used = 0

    def begin(self) -> None:
        ev = self.events[self.turn]
        if ev is not None:
            ev.synchronize()
        self.used = 0

    def take(self, n: int):
        """(host view [n], offset) of the next n elements of this step."""
        off = self.used
        self.used += -(-int(n) // self.ALIGN) * self.ALIGN
        if self.used > self.capacity:
            raise RuntimeError(f"staging buffer too small ({self.used} > {self.capacity})")
        return self.host_np[self.turn][off:off + int(n)], off

    def device(self, off: int, shape) -> torch.Tensor:
        n = int(np.prod(shape))
        return self.dev[off:off + n].view(*shape)

    def commit(self) -> None:
        n = self.used
        if n:
            self.dev[:n].copy_(self.host[self.turn][:n], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record()
            self.events[self.turn] = ev
        self.turn ^= 1


class StepMix:
    """Common driver: subclasses set up sequences and decide who finishes."""

    def __init__(self, spec: workloads.StepMixSpec, draws: workloads.StepDraws,
                 steps: int, max_blocks_per_seq: int, device="cuda",
                 keep_records=False, staging_extra: int = 0, native=False,
                 max_admit_tokens: int = 0, max_groups: int = 0):
        self.spec = spec
        self.draws = draws
        self.steps = int(steps)
        self.mb = int(max_blocks_per_seq)
        self.manager = blocks.BlockManager(spec.num_blocks, spec.block_size,
                                           draws.allocator_seed())
        self.device = device
        torch_dtype = torch.float16 if spec.dtype == np.float16 else torch.float32
        shape = (spec.num_blocks, spec.num_heads, spec.block_size, spec.head_dim)
        self.k_cache = torch.zeros(shape, dtype=torch_dtype, device=device)
        self.v_cache = torch.zeros(shape, dtype=torch_dtype, device=device)
        self.out = torch.empty((spec.num_seqs, spec.num_heads, spec.head_dim),
                               dtype=torch_dtype, device=device)
        self.ws = None
        self.lanes = np.empty(0, dtype=np.int64)  # sequence id of each batch row
        self.records: list[StepRecord] = []
        self.keep = keep_records
        self.next_id = 0
        self.initial = None  # (slots, k, v) written before the first step
        self.copies_total = 0
        self.scale = 1.0 / float(np.sqrt(spec.head_dim))
        self.last_decode = None
        self._inputs: dict[int, StepInputs] = {}
        s = spec.num_seqs
        per_step = 4 * s + s * self.mb + (s + 1) + s + 8 * Staging.ALIGN
        self.staging = Staging(per_step + int(staging_extra), device)
        self._positions = np.empty(s, dtype=np.int32)
        self._last_ctx = None
        # native: each step is one call of the decode-step executor (pa_step.h)
        self.engine = None
        if native:
            from . import engine
            self.engine = engine.StepEngine(self.manager, self.k_cache, self.v_cache, s, self.mb,
                                            max_admit_tokens=max_admit_tokens,
                                            max_groups=max_groups)

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

    def _workspace(self, num_seqs, max_ctx):
        need = ops.pa_decode_workspace_bytes(num_seqs, self.spec.num_heads, self.spec.head_dim,
                                             self.spec.block_size, max_ctx, 0)
        if need and (self.ws is None or self.ws.numel() < need):
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self.ws if need else None

    def _new_id(self) -> int:
        self.next_id += 1
        return self.next_id - 1

    def _admit(self, lens, slots_out: np.ndarray) -> np.ndarray:
        """Admit one sequence per entry of ``lens`` (one native call); their prompt
        slots are written into ``slots_out`` in admission order."""
        ids = np.arange(self.next_id, self.next_id + len(lens), dtype=np.int64)
        self.next_id += len(lens)
        self.manager.add_sequences(ids, lens, slots=slots_out)
        return ids

    def _write_rows(self, slots_d, k_rows, v_rows):
        if slots_d.numel():
            ops.pa_cache_append(self.k_cache, self.v_cache, k_rows, v_rows, slots_d)

    # -- one step -------------------------------------------------------------------
    def _host_extra(self, k_step: int, st: Staging):
        """Subclass hook, run after the decode arrays are staged and before the copy:
        returns a callable that enqueues this step's work after the decode, or None."""
        return None

    def step(self, k_step: int) -> int:
        """Run step ``k_step``; returns the number of sequences decoded."""
        if self.engine is not None:
            return self._native_step(k_step)
        st = self.staging
        st.begin()
        n = len(self.lanes)
        slots_h, o_slots = st.take(n)
        pairs_h, o_pairs = st.take(2 * n)
        tables_h, o_tables = st.take(n * self.mb)
        ctx_h, o_ctx = st.take(n)
        slots, positions, pairs = self.manager.append_slots(
            self.lanes, slots=slots_h, positions=self._positions, pairs=pairs_h.reshape(n, 2))
        tables = self.manager.block_tables(self.lanes, self.mb, out=tables_h.reshape(n, self.mb))
        ctx = self.manager.context_lens(self.lanes, out=ctx_h)
        max_ctx = int(ctx.max())
        self.copies_total += len(pairs)
        if self.keep:
            rec = StepRecord(k_step, pairs.copy(), slots.copy(), None, None, positions.copy(),
                             tables.copy(), ctx.copy(), None)
        decode = self._decode_call(k_step, st, tables, ctx, o_tables, o_ctx, max_ctx)
        after = self._host_extra(k_step, st)
        st.commit()

        inp = self.inputs(k_step)
        nk_d, nv_d, q_d = inp.dev[:3] if inp.dev else (self.to_dev(inp.new_k),
                                                        self.to_dev(inp.new_v),
                                                        self.to_dev(inp.q))
        if len(pairs):
            ops.pa_block_copy(self.k_cache, self.v_cache, st.device(o_pairs, (len(pairs), 2)))
        self._write_rows(st.device(o_slots, (n,)), nk_d, nv_d)
        self.last_decode = lambda: decode(q_d)
        self.last_decode()
        if after is not None:
            after()
        if self.keep:
            rec.new_k, rec.new_v, rec.q = inp.new_k, inp.new_v, inp.q
            self._finish_record(rec)
            self.records.append(rec)
        self._last_ctx = ctx
        return n

    def last_context_lens(self) -> np.ndarray:
        """Context lengths of the last step's sequences (the new token counted)."""
        if self.engine is not None:
            return self.engine.last()["context_lens"]
        return np.array(self._last_ctx)

    # -- one step through the native executor -----------------------------------------
    def _native_requests(self, k_step: int, inp: StepInputs) -> dict:
        """Subclass hook: finished sequences and admission requests of the step."""
        return {}

    def _native_groups(self):
        """Subclass hook: group_starts of a shared-prefix decode, or None."""
        return None

    def _native_step(self, k_step: int) -> int:
        inp = self.inputs(k_step)
        nk_d, nv_d, q_d = inp.dev[:3] if inp.dev else (self.to_dev(inp.new_k),
                                                        self.to_dev(inp.new_v),
                                                        self.to_dev(inp.q))
        req = self._native_requests(k_step, inp)
        groups = self._native_groups()
        n = len(self.lanes)
        res = self.engine.run(self.lanes, q_d, nk_d, nv_d, self.out, self.scale,
                              group_starts=groups, **req)
        self.copies_total += res.num_copies
        if "admit_ids" in req:
            if res.num_admitted != len(req["admit_ids"]):
                raise blocks.OutOfBlocks(f"{res.num_admitted} of {len(req['admit_ids'])} "
                                         "requests admitted")
            self.lanes[inp.finishing] = req["admit_ids"]
        if self.keep:
            v = self.engine.last()
            rec = StepRecord(k_step, v["copy_pairs"], v["slots"], inp.new_k, inp.new_v,
                             v["positions"], v["block_tables"], v["context_lens"], inp.q)
            if v["admit_slots"].size:
                rec.post_slots, rec.post_k, rec.post_v = v["admit_slots"], inp.prompt_k, inp.prompt_v
            if groups is not None:
                self.last_prefix = (v["group_starts"], v["prefix_lens"])
            self.records.append(rec)
        self.last_decode = lambda: self.engine.decode_again(q_d, self.out, self.scale)
        return n

    def _finish_record(self, rec: StepRecord) -> None:
        pass

    # the executor's launch hints for pa_decode: 8-wave workgroups, and the longest
    # contexts first unless the batch's sequences share blocks (include/pa_step.h)
    ORDER_LONGEST_FIRST = True

    def _decode_call(self, k_step, st, tables, ctx, o_tables, o_ctx, max_ctx):
        """The step's decode as a callable of the query (enqueued once per step, and
        again for timing)."""
        n = len(self.lanes)
        tables_d = st.device(o_tables, (n, self.mb))
        ctx_d = st.device(o_ctx, (n,))
        ws = self._workspace(n, max_ctx)
        order_d = None
        if self.ORDER_LONGEST_FIRST:
            order_h, o_order = st.take(n)
            order_h[:] = np.argsort(-np.asarray(ctx), kind="stable")
            order_d = st.device(o_order, (n,))

        def call(q_d):
            ops.pa_decode(self.out, q_d, self.k_cache, self.v_cache, tables_d, ctx_d,
                          self.scale, max_ctx, 0, ws, seq_order=order_d,
                          waves=ops.DECODE_WAVES_NARROW)
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
                 keep_records=False, native=False):
        spec = workloads.CONTINUOUS_BATCHING
        draws = workloads.ContinuousBatchingDraws(spec, seed)
        steps = steps or spec.steps
        mb = -(-(draws.prompt_high + steps) // spec.block_size)
        prompt_room = draws.finish_count * draws.prompt_high + Staging.ALIGN
        super().__init__(spec, draws, steps, mb, device, keep_records, staging_extra=prompt_room,
                         native=native, max_admit_tokens=prompt_room)
        lens = draws.initial_prompt_lens()
        k, v = draws.prompt_kv(-1, lens)
        slots = np.empty(int(lens.sum()) + 1, dtype=np.int32)
        self.lanes = np.array(self._admit(lens, slots), dtype=np.int64)
        slots = slots[:int(lens.sum())]
        ops.pa_cache_append(self.k_cache, self.v_cache, self.to_dev(k), self.to_dev(v),
                            self.to_dev(slots))
        self.initial = (slots, k, v)
        self._post = None

    def _draw_inputs(self, k: int) -> StepInputs:
        inp = super()._draw_inputs(k)
        inp.prompt_lens = self.draws.replacement_prompt_lens(k)
        inp.finishing = self.draws.finishing(k)
        inp.prompt_k, inp.prompt_v = self.draws.prompt_kv(k, inp.prompt_lens)
        return inp

    def _host_extra(self, k_step: int, st: Staging):
        # admit, then retire (as the executor does): the new prompts take only blocks
        # that were free before this step, and the finished sequences' blocks serve
        # the next step's admissions
        inp = self.inputs(k_step)
        finishing = inp.finishing
        total = int(inp.prompt_lens.sum())
        pslots_h, o_p = st.take(total + 1)
        ids = self._admit(inp.prompt_lens, pslots_h)
        for lane in finishing:
            self.manager.free(int(self.lanes[lane]))
        self.lanes[finishing] = ids
        self._post = pslots_h[:total].copy() if self.keep else None
        pslots_d = st.device(o_p, (total,))
        k_dev, v_dev = inp.dev[3:] if inp.dev else (self.to_dev(inp.prompt_k),
                                                     self.to_dev(inp.prompt_v))
        return lambda: self._write_rows(pslots_d, k_dev, v_dev)

    def _finish_record(self, rec: StepRecord) -> None:
        inp = self.inputs(rec.step)
        rec.post_slots, rec.post_k, rec.post_v = self._post, inp.prompt_k, inp.prompt_v

    def _native_requests(self, k_step: int, inp: StepInputs) -> dict:
        ids = np.arange(self.next_id, self.next_id + len(inp.prompt_lens), dtype=np.int64)
        self.next_id += len(ids)
        k_dev, v_dev = inp.dev[3:] if inp.dev else (self.to_dev(inp.prompt_k),
                                                     self.to_dev(inp.prompt_v))
        return {"finished": self.lanes[inp.finishing], "admit_ids": ids,
                "admit_lens": inp.prompt_lens, "prompt_key": k_dev, "prompt_value": v_dev}

    def run_step(self, k_step: int):
        return self.step(k_step)


class SharedPrefix(StepMix):
    """8 groups x 8 samples sharing their prompt blocks (see module docstring).

    With ``shared_decode`` the decode runs through pa_decode_shared_prefix: each
    group's leading blocks that all of its samples still hold are read once for the
    whole group."""

    ORDER_LONGEST_FIRST = False  # the samples share blocks: keep each group together

    def __init__(self, seed: int, steps: int | None = None, device="cuda",
                 keep_records=False, shared_decode=False, native=False):
        self.shared_decode = bool(shared_decode)
        self.ws_shared = None
        spec = workloads.SHARED_PREFIX
        draws = workloads.SharedPrefixDraws(spec, seed)
        steps = steps or spec.steps
        lens = draws.prompt_lens()
        mb = -(-(int(lens.max()) + steps) // spec.block_size)
        super().__init__(spec, draws, steps, mb, device, keep_records, native=native,
                         max_groups=spec.num_seqs)
        k, v = draws.prompt_kv(-1, lens)
        slots = np.empty(int(lens.sum()) + 1, dtype=np.int32)
        leaders = self._admit(lens, slots)
        slots = slots[:int(lens.sum())]
        lanes = []
        for leader in leaders:
            lanes.append(leader)
            for _ in range(draws.samples - 1):
                child = self._new_id()
                self.manager.fork(leader, child)
                lanes.append(child)
        self.lanes = np.array(lanes, dtype=np.int64)
        ops.pa_cache_append(self.k_cache, self.v_cache, self.to_dev(k), self.to_dev(v),
                            self.to_dev(slots))
        self.initial = (slots, k, v)

    def shared_prefix(self):
        """(group_starts, prefix_lens) of the running lanes: a group is 8 contiguous
        lanes; its prefix is the leading whole blocks all of its members hold."""
        n = self.draws.samples
        starts = np.arange(0, len(self.lanes) + 1, n, dtype=np.int32)
        prefix = np.zeros(len(self.lanes), dtype=np.int32)
        for r0 in starts[:-1]:
            prefix[r0:r0 + n] = (self.manager.shared_prefix_blocks(self.lanes[r0:r0 + n]) *
                                 self.spec.block_size)
        return starts, prefix

    def _native_groups(self):
        if not self.shared_decode:
            return None
        return np.arange(0, len(self.lanes) + 1, self.draws.samples, dtype=np.int32)

    def _decode_call(self, k_step, st, tables, ctx, o_tables, o_ctx, max_ctx):
        if not self.shared_decode:
            return super()._decode_call(k_step, st, tables, ctx, o_tables, o_ctx, max_ctx)
        n = len(self.lanes)
        starts, prefix = self.shared_prefix()
        starts_h, o_starts = st.take(len(starts))
        prefix_h, o_prefix = st.take(n)
        starts_h[:] = starts
        prefix_h[:] = prefix
        self.last_prefix = (starts, prefix)
        max_prefix = int(prefix.max())
        max_suffix = int((ctx - prefix).max())
        tables_d = st.device(o_tables, (n, self.mb))
        ctx_d = st.device(o_ctx, (n,))
        starts_d = st.device(o_starts, (len(starts),))
        prefix_d = st.device(o_prefix, (n,))
        largest = int(np.diff(starts).max())
        need = ops.pa_decode_shared_prefix_workspace_bytes(
            n, self.spec.num_heads, self.spec.head_dim, self.spec.block_size, len(starts) - 1,
            max_prefix, max_suffix, max_group_size=largest)
        if self.ws_shared is None or self.ws_shared.numel() < need:
            self.ws_shared = torch.empty(need, dtype=torch.uint8, device=self.device)
        ws = self.ws_shared

        def call(q_d):
            ops.pa_decode_shared_prefix(self.out, q_d, self.k_cache, self.v_cache, tables_d,
                                        ctx_d, starts_d, prefix_d, self.scale, max_prefix,
                                        max_suffix, workspace=ws, max_group_size=largest)
        return call

    def run_step(self, k_step: int):
        return self.step(k_step)
