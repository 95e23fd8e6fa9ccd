"""Python binding of the decode-step executor of ``libpa.so`` (include/pa_step.h).

One :meth:`StepEngine.run` is one native call for a whole decode step: the block
manager reserves every running sequence's next slot (fresh block or copy-on-write),
the step's tables and lengths go to the device in one copy from pinned memory, and
the block copy, the append of the new K/V rows and the decode are enqueued on the
current stream; finished sequences give their blocks back and waiting requests are
admitted (their prompt rows written after the decode) in the same call.  The order
follows the request life cycle of "vLLM基础：架构、推理流程与关键组件" §2.2 and the
scheduler step of "啃透vLLM源码：从PagedAttention到连续批处理，大模型推理加速24倍的秘密" §3.

Argument marshalling only, like :mod:`ops`: the device arrays' shapes are checked
here (the library cannot see them), everything else runs in the library.
"""

from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import blocks, ops

_i32, _f32, _vp = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
_p32 = ctypes.POINTER(ctypes.c_int32)


class _Config(ctypes.Structure):
    _fields_ = [("num_heads", _i32), ("head_dim", _i32), ("dtype", _i32), ("max_seqs", _i32),
                ("max_blocks_per_seq", _i32), ("max_admit_tokens", _i32), ("max_groups", _i32)]


class _Args(ctypes.Structure):
    _fields_ = [("seq_ids", _vp), ("num_seqs", _i32), ("query", _vp), ("new_key", _vp),
                ("new_value", _vp), ("out", _vp), ("scale", _f32), ("group_starts", _vp),
                ("num_groups", _i32), ("finished_ids", _vp), ("num_finished", _i32),
                ("admit_ids", _vp), ("admit_lens", _vp), ("num_admit", _i32),
                ("prompt_key", _vp), ("prompt_value", _vp)]


class StepResult(ctypes.Structure):
    _fields_ = [("num_copies", _i32), ("num_admitted", _i32), ("admitted_tokens", _i32),
                ("max_context_len", _i32), ("max_prefix_len", _i32), ("max_suffix_len", _i32),
                ("max_group_size", _i32)]


class _View(ctypes.Structure):
    _fields_ = [("num_seqs", _i32), ("num_groups", _i32), ("result", StepResult),
                ("slots", _p32), ("positions", _p32), ("copy_pairs", _p32),
                ("block_tables", _p32), ("context_lens", _p32), ("group_starts", _p32),
                ("prefix_lens", _p32), ("admit_slots", _p32), ("dev_block_tables", _vp),
                ("dev_context_lens", _vp), ("dev_group_starts", _vp), ("dev_prefix_lens", _vp),
                ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
                ("hints", ops.DecodeHints)]


def _host_array(ptr, shape) -> np.ndarray:
    if not ptr or int(np.prod(shape)) == 0:
        return np.zeros(shape, dtype=np.int32)
    return np.ctypeslib.as_array(ptr, shape=shape).copy()


def _ids(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64).reshape(-1))


class StepEngine:
    """Decode steps over ``manager`` and the pools ``key_cache`` / ``value_cache``
    ([num_blocks, H, block_size, D] on one GPU), for up to ``max_seqs`` running
    sequences of at most ``max_blocks_per_seq`` blocks, ``max_admit_tokens`` prompt
    tokens requested per step and ``max_groups`` shared-prefix groups."""

    def __init__(self, manager: blocks.BlockManager, key_cache: torch.Tensor,
                 value_cache: torch.Tensor, max_seqs: int, max_blocks_per_seq: int,
                 max_admit_tokens: int = 0, max_groups: int = 0):
        self._lib = ops.lib
        self._h = None
        nb, h, bs, d = key_cache.shape
        if value_cache.shape != key_cache.shape or value_cache.dtype != key_cache.dtype:
            raise ValueError("key and value pools differ")
        if (nb, bs) != (manager.num_blocks, manager.block_size):
            raise ValueError(f"pools hold {nb} blocks of {bs}, the manager "
                             f"{manager.num_blocks} of {manager.block_size}")
        if not (key_cache.is_contiguous() and value_cache.is_contiguous()):
            raise ValueError("pools must be contiguous")
        self.device = ops._same_device(key_cache, value_cache)
        self.dtype = key_cache.dtype
        self.num_heads, self.head_dim, self.block_size = h, d, bs
        self.max_seqs = int(max_seqs)
        self.max_blocks_per_seq = int(max_blocks_per_seq)
        self.max_admit_tokens = int(max_admit_tokens)
        # the manager and the pools must outlive the executor
        self.manager, self.key_cache, self.value_cache = manager, key_cache, value_cache
        cfg = _Config(h, d, ops._dtype(key_cache), self.max_seqs, self.max_blocks_per_seq,
                      self.max_admit_tokens, int(max_groups))
        with torch.cuda.device(self.device):
            self._h = self._lib.pa_step_create(manager._h, ctypes.byref(cfg),
                                               key_cache.data_ptr(), value_cache.data_ptr())
        if not self._h:
            raise ops.PagedAttentionError(2, self._lib.pa_last_error().decode())
        self._args = _Args()
        self._res = StepResult()
        self._view = _View()
        self._row_shape = (h, d)

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            self._lib.pa_step_destroy(h)

    def _rows(self, t: torch.Tensor, n: int, name: str, at_least=False) -> int:
        ok = (t.dtype == self.dtype and t.dim() == 3 and tuple(t.shape[1:]) == self._row_shape
              and (t.shape[0] >= n if at_least else t.shape[0] == n) and t.is_contiguous()
              and t.get_device() == self.device)
        if not ok:
            raise ValueError(f"{name} must be a contiguous {self.dtype} tensor [{n}, "
                             f"{self._row_shape[0]}, {self._row_shape[1]}] on cuda:{self.device}")
        return t.data_ptr()

    def run(self, seq_ids: np.ndarray, query, new_key, new_value, out, scale: float,
            group_starts: np.ndarray | None = None, finished: np.ndarray | None = None,
            admit_ids: np.ndarray | None = None, admit_lens: np.ndarray | None = None,
            prompt_key=None, prompt_value=None, stream=None) -> StepResult:
        """One decode step (include/pa_step.h); returns its counts.  ``seq_ids``,
        ``finished`` and ``admit_ids`` are int64 arrays, ``group_starts`` and
        ``admit_lens`` int32 arrays (host); the tensors are device arrays."""
        a = self._args
        seq_ids = _ids(seq_ids)
        n = seq_ids.size
        a.seq_ids, a.num_seqs = seq_ids.ctypes.data, n
        a.query = self._rows(query, n, "query")
        a.new_key = self._rows(new_key, n, "new_key")
        a.new_value = self._rows(new_value, n, "new_value")
        a.out = self._rows(out, n, "out")
        a.scale = float(scale)
        if group_starts is not None:
            group_starts = np.ascontiguousarray(group_starts, dtype=np.int32)
            a.group_starts, a.num_groups = group_starts.ctypes.data, group_starts.size - 1
        else:
            a.group_starts, a.num_groups = None, 0
        if finished is not None and len(finished):
            finished = _ids(finished)
            a.finished_ids, a.num_finished = finished.ctypes.data, finished.size
        else:
            a.finished_ids, a.num_finished = None, 0
        if admit_ids is not None and len(admit_ids):
            admit_ids = _ids(admit_ids)
            admit_lens = np.ascontiguousarray(admit_lens, dtype=np.int32).reshape(-1)
            if admit_lens.size != admit_ids.size:
                raise ValueError("admit_ids and admit_lens differ in length")
            total = int(admit_lens.sum())
            a.admit_ids, a.admit_lens, a.num_admit = (admit_ids.ctypes.data,
                                                      admit_lens.ctypes.data, admit_ids.size)
            if total:
                a.prompt_key = self._rows(prompt_key, total, "prompt_key", at_least=True)
                a.prompt_value = self._rows(prompt_value, total, "prompt_value", at_least=True)
            else:
                a.prompt_key = a.prompt_value = None
        else:
            a.admit_ids, a.admit_lens, a.num_admit = None, None, 0
            a.prompt_key = a.prompt_value = None
        status = self._lib.pa_step_run(self._h, ctypes.byref(a), ops._stream(stream, self.device),
                                       ctypes.byref(self._res))
        if status != 0:
            msg = self._lib.pa_last_error().decode()
            if status == 6:
                raise blocks.OutOfBlocks(msg)
            raise ops.PagedAttentionError(status, msg)
        return self._res

    def _last_view(self) -> _View:
        ops._check(self._lib.pa_step_last(self._h, ctypes.byref(self._view)))
        return self._view

    def last(self) -> dict:
        """Copies of the host arrays of the last step: slots, positions, copy_pairs,
        block_tables, context_lens, group_starts, prefix_lens, admit_slots, and its
        counts."""
        v = self._last_view()
        n, r = v.num_seqs, v.result
        grouped = v.num_groups > 0
        return {
            "slots": _host_array(v.slots, (n,)),
            "positions": _host_array(v.positions, (n,)),
            "copy_pairs": _host_array(v.copy_pairs, (r.num_copies, 2)),
            "block_tables": _host_array(v.block_tables, (n, self.max_blocks_per_seq)),
            "context_lens": _host_array(v.context_lens, (n,)),
            "group_starts": _host_array(v.group_starts, (v.num_groups + 1,)) if grouped else None,
            "prefix_lens": _host_array(v.prefix_lens, (n,)) if grouped else None,
            "admit_slots": _host_array(v.admit_slots, (r.admitted_tokens,)),
            "num_copies": r.num_copies, "num_admitted": r.num_admitted,
            "max_context_len": r.max_context_len, "max_prefix_len": r.max_prefix_len,
            "max_suffix_len": r.max_suffix_len, "max_group_size": r.max_group_size,
        }

    def decode_again(self, query, out, scale: float, stream=None) -> None:
        """Enqueue the last step's decode once more with its device arrays (valid until
        the next step; e.g. to time the decode alone)."""
        v = self._last_view()
        n, r = v.num_seqs, v.result
        q = self._rows(query, n, "query")
        o = self._rows(out, n, "out")
        h, d = self._row_shape
        nb = self.manager.num_blocks
        dt = ops._dtype(query)
        s = ops._stream(stream, self.device)
        kc, vc = self.key_cache.data_ptr(), self.value_cache.data_ptr()
        if v.num_groups > 0:
            status = self._lib.pa_decode_shared_prefix(
                o, q, kc, vc, v.dev_block_tables, v.dev_context_lens, v.dev_group_starts,
                v.dev_prefix_lens, n, h, d, self.block_size, nb, self.max_blocks_per_seq,
                v.num_groups, r.max_group_size, r.max_prefix_len, r.max_suffix_len, float(scale),
                dt, 0, 0, v.workspace, v.workspace_bytes, s)
        else:  # with the step's own launch hints (workgroup size, dispatch order)
            status = self._lib.pa_decode_ex(o, q, kc, vc, v.dev_block_tables, v.dev_context_lens, n,
                                            h, d, self.block_size, nb, self.max_blocks_per_seq,
                                            r.max_context_len, float(scale), dt, 0, v.workspace,
                                            v.workspace_bytes, ctypes.byref(v.hints), s)
        ops._check(status)
