"""Python binding of ``libpa.so``: the C-ABI entry points under the same names.

Argument marshalling only: shapes are read from the tensors, pointers and the
current HIP stream are passed through, and a non-OK status raises
:class:`PagedAttentionError` with the library's message.  Every step of the path
runs in the HIP kernels; there is no fallback.  Importing this module loads the
library and raises if it has not been built.
"""

from __future__ import annotations

import ctypes
import pathlib

import torch

LIB_PATH = pathlib.Path(__file__).resolve().with_name("libpa.so")
# the same kernels with every entry point checking its device data first (pa.h)
DEBUG_LIB_PATH = LIB_PATH.with_name("libpa_debug.so")

PA_F32 = 0
PA_F16 = 1
PA_NOALLOC_SCRATCH_BYTES = 32 << 20  # size of pa_decode_noalloc's scratch array (pa.h)
DECODE_WAVES_NARROW, DECODE_WAVES_WIDE = 8, 16  # the two decode workgroup sizes
_DTYPES = {torch.float32: PA_F32, torch.float16: PA_F16}
_STATUS = {0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_INVALID_ARG", 3: "PA_ERR_UNSUPPORTED",
           4: "PA_ERR_WORKSPACE", 5: "PA_ERR_HIP", 6: "PA_ERR_OUT_OF_BLOCKS"}

# name -> (restype, argtypes), mirroring include/pa.h
_i32, _f32, _sz, _vp = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
SIGNATURES = {
    "pa_abi_version": (_i32, []),
    "pa_debug_checks": (_i32, []),
    "pa_status_string": (ctypes.c_char_p, [_i32]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_decode_partition_size": (_i32, [_i32, _i32, _i32, _i32, _i32]),
    "pa_decode_num_partitions": (_i32, [_i32, _i32, _i32, _i32, _i32]),
    "pa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_waves": (_i32, [_i32] * 7),
    "pa_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                         _i32, _f32, _i32, _i32, _vp, _sz, _vp]),
    "pa_decode_append": (_i32, [_vp] * 8 + [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                                             _i32, _vp, _sz, _vp]),
    "pa_decode_ex": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                            _i32, _f32, _i32, _i32, _vp, _sz, _vp, _vp]),
    "pa_decode_append_ex": (_i32, [_vp] * 8 + [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                                _i32, _i32, _vp, _sz, _vp, _vp]),
    "pa_decode_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                 _i32, _i32, _f32, _i32, _i32, _vp]),
    "pa_decode_partitions": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                    _i32, _i32, _i32, _f32, _i32, _i32, _vp, _sz, _vp]),
    "pa_decode_reduce": (_i32, [_vp, _vp, _sz, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                _vp]),
    "pa_cache_append": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                               _vp]),
    "pa_block_copy": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pa_decode_shared_prefix_workspace_bytes": (_sz, [_i32] * 10),
    "pa_swap_blocks": (_i32, [_vp] * 5 + [_i32] * 7 + [_vp]),
    # host block manager (include/pa_blocks.h)
    "pa_bm_create": (_vp, [_i32, _i32, ctypes.c_uint64]),
    "pa_bm_destroy": (None, [_vp]),
    "pa_bm_num_blocks": (_i32, [_vp]),
    "pa_bm_block_size": (_i32, [_vp]),
    "pa_bm_num_free": (_i32, [_vp]),
    "pa_bm_can_allocate": (_i32, [_vp, _i32]),
    "pa_bm_ref_counts": (_i32, [_vp, _vp]),
    "pa_bm_add_sequence": (_i32, [_vp, ctypes.c_int64, _i32, _vp]),
    "pa_bm_add_sequences": (_i32, [_vp, _vp, _vp, _i32, _vp]),
    "pa_bm_fork": (_i32, [_vp, ctypes.c_int64, ctypes.c_int64]),
    "pa_bm_free": (_i32, [_vp, ctypes.c_int64]),
    "pa_bm_append_slots": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp]),
    "pa_bm_block_tables": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp]),
    "pa_bm_context_lens": (_i32, [_vp, _vp, _i32, _vp]),
    "pa_bm_shared_prefix_blocks": (_i32, [_vp, _vp, _i32]),
    "pa_bm_num_seq_blocks": (_i32, [_vp, ctypes.c_int64]),
    "pa_bm_seq_blocks": (_i32, [_vp, ctypes.c_int64, _vp, _i32]),
    "pa_decode_shared_prefix": (_i32, [_vp] * 8 + [_i32] * 10 + [_f32, _i32, _i32, _i32, _vp,
                                                                 _sz, _vp]),
    # decode-step executor (include/pa_step.h); structs are passed by pointer
    "pa_step_create": (_vp, [_vp, _vp, _vp, _vp]),
    "pa_step_destroy": (None, [_vp]),
    "pa_step_run": (_i32, [_vp, _vp, _vp, _vp]),
    "pa_step_last": (_i32, [_vp, _vp]),
}


class DecodeHints(ctypes.Structure):
    """pa_decode_hints of include/pa.h: a dispatch order and a workgroup size."""
    _fields_ = [("seq_order", _vp), ("waves", _i32)]


def _hints(seq_order, waves, device):
    """A DecodeHints for the call, or None when neither hint is given."""
    if seq_order is None and not waves:
        return None
    if seq_order is not None:
        _int32(seq_order)
        if seq_order.dim() != 1 or seq_order.get_device() != device:
            raise ValueError("seq_order must be a 1-D int32 tensor on the call's GPU")
    return ctypes.byref(DecodeHints(_ptr(seq_order) if seq_order is not None else None, int(waves)))


class PagedAttentionError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def load_library(path: pathlib.Path | str = LIB_PATH) -> ctypes.CDLL:
    path = pathlib.Path(path)
    if not path.exists():
        raise RuntimeError(
            f"{path} is missing: build it with `python -m paged_kv_cache_414_amd.build`")
    lib = ctypes.CDLL(str(path))
    for name, (restype, argtypes) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = restype
        fn.argtypes = argtypes
    return lib


lib = load_library()


def _check(status: int) -> None:
    if status != 0:
        raise PagedAttentionError(status, lib.pa_last_error().decode())


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libpa must be contiguous")
    return t.data_ptr() if t.numel() else None


try:  # the current stream's raw handle without building a Stream object
    _raw_stream = torch._C._cuda_getCurrentRawStream
except AttributeError:  # pragma: no cover
    _raw_stream = None


def _stream(stream, device) -> int | None:
    if stream is None:
        index = device if isinstance(device, int) else device.index
        if _raw_stream is not None:
            return _raw_stream(index)
        stream = torch.cuda.current_stream(index)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype} (float32 or float16)") from None


def _same_device(*ts) -> int:
    """Index of the one GPU all tensors live on."""
    devs = {t.get_device() for t in ts if t is not None}
    if len(devs) != 1 or next(iter(devs)) < 0:
        raise ValueError(f"all tensors must be on one GPU, got {[t.device for t in ts if t is not None]}")
    return next(iter(devs))


def _int32(*ts):
    for t in ts:
        if t.dtype != torch.int32:
            raise ValueError("index tensors must be int32")


# ----------------------------------------------------------------------------------
# planning
# ----------------------------------------------------------------------------------

def pa_decode_partition_size(num_seqs, num_heads, block_size, max_context_len,
                             partition_size=0) -> int:
    p = lib.pa_decode_partition_size(num_seqs, num_heads, block_size, max_context_len,
                                     partition_size)
    if p < 0:
        raise PagedAttentionError(2, lib.pa_last_error().decode())
    return p


def pa_decode_num_partitions(num_seqs, num_heads, block_size, max_context_len,
                             partition_size=0) -> int:
    n = lib.pa_decode_num_partitions(num_seqs, num_heads, block_size, max_context_len,
                                     partition_size)
    if n < 0:
        raise PagedAttentionError(2, lib.pa_last_error().decode())
    return n


def pa_decode_waves(num_seqs, num_heads, head_dim, block_size, max_context_len,
                    partition_size=0, dtype=torch.float16) -> int:
    """Wave64s per workgroup of pa_decode's partition pass for these arguments."""
    w = lib.pa_decode_waves(num_seqs, num_heads, head_dim, block_size, max_context_len,
                            partition_size, _DTYPES[dtype])
    if w < 0:
        raise PagedAttentionError(2, lib.pa_last_error().decode())
    return w


def pa_decode_workspace_bytes(num_seqs, num_heads, head_dim, block_size, max_context_len,
                              partition_size=0) -> int:
    return int(lib.pa_decode_workspace_bytes(num_seqs, num_heads, head_dim, block_size,
                                             max_context_len, partition_size))


def workspace_for(query: torch.Tensor, key_cache: torch.Tensor, max_context_len: int,
                  partition_size: int = 0) -> torch.Tensor | None:
    """Device buffer of the size pa_decode needs (None when none is needed)."""
    s, h, d = query.shape
    n = pa_decode_workspace_bytes(s, h, d, key_cache.shape[2], max_context_len,
                                  partition_size)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=query.device)


# ----------------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------------

def _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                 max_context_len, partition_size, workspace, stream):
    dev = _same_device(out, query, key_cache, value_cache, block_tables, context_lens)
    _int32(block_tables, context_lens)
    if not (out.dtype == query.dtype == key_cache.dtype == value_cache.dtype):
        raise ValueError("out, query and the caches must share one dtype")
    s, h, d = query.shape
    nb, hk, bs, dk = key_cache.shape
    if (hk, dk) != (h, d) or value_cache.shape != key_cache.shape or out.shape != query.shape:
        raise ValueError("shape mismatch between query/out [S,H,D] and caches [NB,H,bs,D]")
    if block_tables.dim() != 2 or block_tables.shape[0] != s or context_lens.shape != (s,):
        raise ValueError("block_tables must be [S, MB] and context_lens [S]")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return (_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
            _ptr(context_lens), s, h, d, bs, nb, block_tables.shape[1], int(max_context_len),
            float(scale), _dtype(query), int(partition_size), _ptr(workspace), ws_bytes,
            _stream(stream, dev))


def pa_decode(out, query, key_cache, value_cache, block_tables, context_lens, scale,
              max_context_len, partition_size=0, workspace=None, stream=None, seq_order=None,
              waves=0):
    """Paged decode attention into ``out`` [S, H, D] (see include/pa.h).  With
    ``seq_order`` (int32 [S] on the GPU, a permutation) or ``waves`` (8 or 16) the call
    is pa_decode_ex with those launch hints."""
    args = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                        max_context_len, partition_size, workspace, stream)
    hints = _hints(seq_order, waves, query.get_device())
    if hints is None:
        _check(lib.pa_decode(*args))
    else:
        _check(lib.pa_decode_ex(*args[:-1], hints, args[-1]))
    return out


def pa_decode_noalloc(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                      max_context_len, partition_size=0, stream=None):
    """pa_decode with the partition states in the library's own scratch array instead
    of a caller workspace (see include/pa.h: for callers that cannot allocate)."""
    args = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                        max_context_len, partition_size, None, stream)
    _check(lib.pa_decode_noalloc(*args[:16], args[18]))
    return out


def pa_decode_append(out, query, key_cache, value_cache, new_key, new_value, block_tables,
                     context_lens, scale, max_context_len, partition_size=0, workspace=None,
                     stream=None, seq_order=None, waves=0):
    """Append each sequence's newest K/V row ``new_key`` / ``new_value`` [S, H, D] at
    position context_lens[s] - 1, then paged decode attention into ``out``, in one
    call (see include/pa.h); with launch hints as :func:`pa_decode`."""
    args = _decode_args(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                        max_context_len, partition_size, workspace, stream)
    _same_device(query, new_key, new_value)
    for name, t in (("new_key", new_key), ("new_value", new_value)):
        if t.dtype != query.dtype or t.shape != query.shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {query.dtype} tensor shaped like query")
    hints = _hints(seq_order, waves, query.get_device())
    if hints is None:
        _check(lib.pa_decode_append(*args[:4], _ptr(new_key), _ptr(new_value), *args[4:]))
    else:
        _check(lib.pa_decode_append_ex(*args[:4], _ptr(new_key), _ptr(new_value), *args[4:-1],
                                       hints, args[-1]))
    return out


def pa_decode_partitions(out, query, key_cache, value_cache, block_tables, context_lens,
                         scale, max_context_len, partition_size=0, workspace=None,
                         stream=None):
    """First (partition) pass of pa_decode alone."""
    _check(lib.pa_decode_partitions(*_decode_args(out, query, key_cache, value_cache,
                                                  block_tables, context_lens, scale,
                                                  max_context_len, partition_size,
                                                  workspace, stream)))
    return out


def pa_decode_reduce(out, workspace, context_lens, block_size, max_context_len,
                     partition_size=0, stream=None):
    """Second (merge) pass of pa_decode alone."""
    dev = _same_device(out, context_lens)
    _int32(context_lens)
    s, h, d = out.shape
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.pa_decode_reduce(_ptr(out), _ptr(workspace), ws_bytes, _ptr(context_lens), s,
                                h, d, int(block_size), int(max_context_len), _dtype(out),
                                int(partition_size), _stream(stream, dev)))
    return out


def pa_cache_append(key_cache, value_cache, key, value, slot_mapping, stream=None):
    """Write key/value rows [T, H, D] into the caches at ``slot_mapping`` [T]."""
    dev = _same_device(key_cache, value_cache, key, value, slot_mapping)
    _int32(slot_mapping)
    if not (key_cache.dtype == value_cache.dtype == key.dtype == value.dtype):
        raise ValueError("caches and key/value must share one dtype")
    nb, h, bs, d = key_cache.shape
    t = key.shape[0]
    if key.shape != (t, h, d) or value.shape != key.shape or slot_mapping.shape != (t,):
        raise ValueError("key/value must be [T, H, D] and slot_mapping [T]")
    if value_cache.shape != key_cache.shape:
        raise ValueError("key and value caches differ in shape")
    _check(lib.pa_cache_append(_ptr(key_cache), _ptr(value_cache), _ptr(key), _ptr(value),
                               _ptr(slot_mapping), t, h, d, bs, nb, _dtype(key),
                               _stream(stream, dev)))


def pa_block_copy(key_cache, value_cache, block_pairs, stream=None):
    """Copy whole blocks: for each row (src, dst) of ``block_pairs`` [n, 2]."""
    dev = _same_device(key_cache, value_cache, block_pairs)
    _int32(block_pairs)
    nb, h, bs, d = key_cache.shape
    if block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [n, 2]")
    if value_cache.shape != key_cache.shape or value_cache.dtype != key_cache.dtype:
        raise ValueError("key and value caches differ")
    _check(lib.pa_block_copy(_ptr(key_cache), _ptr(value_cache), _ptr(block_pairs),
                             block_pairs.shape[0], h, d, bs, nb, _dtype(key_cache),
                             _stream(stream, dev)))


# ----------------------------------------------------------------------------------
# shared-prefix decode
# ----------------------------------------------------------------------------------

def pa_decode_shared_prefix_workspace_bytes(num_seqs, num_heads, head_dim, block_size,
                                            num_groups, max_prefix_len, max_suffix_len,
                                            partition_size=0, prefix_partition_size=0,
                                            max_group_size=0) -> int:
    n = int(lib.pa_decode_shared_prefix_workspace_bytes(
        num_seqs, num_heads, head_dim, block_size, num_groups, int(max_group_size),
        max_prefix_len, max_suffix_len, partition_size, prefix_partition_size))
    if n == 0 and num_seqs > 0:
        raise PagedAttentionError(2, lib.pa_last_error().decode())
    return n


def shared_prefix_workspace_for(query, key_cache, num_groups, max_prefix_len,
                                max_suffix_len, partition_size=0,
                                prefix_partition_size=0, max_group_size=0) -> torch.Tensor | None:
    """Device buffer of the size pa_decode_shared_prefix needs."""
    s, h, d = query.shape
    n = pa_decode_shared_prefix_workspace_bytes(s, h, d, key_cache.shape[2], num_groups,
                                                max_prefix_len, max_suffix_len,
                                                partition_size, prefix_partition_size,
                                                max_group_size)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=query.device)


def pa_decode_shared_prefix(out, query, key_cache, value_cache, block_tables, context_lens,
                            group_starts, prefix_lens, scale, max_prefix_len, max_suffix_len,
                            partition_size=0, prefix_partition_size=0, workspace=None,
                            stream=None, max_group_size=0):
    """pa_decode for groups of sequences that share leading blocks (see include/pa.h).

    group_starts int32 [G + 1] and prefix_lens int32 [S] describe the groups;
    max_group_size (members of the largest group, 0 = library choice) sizes the launch
    and must match the value the workspace was sized with."""
    args = list(_decode_args(out, query, key_cache, value_cache, block_tables, context_lens,
                             scale, 0, partition_size, workspace, stream))
    dev = _same_device(out, group_starts, prefix_lens)
    _int32(group_starts, prefix_lens)
    s = query.shape[0]
    if group_starts.dim() != 1 or prefix_lens.shape != (s,):
        raise ValueError("group_starts must be [G + 1] and prefix_lens [S]")
    num_groups = group_starts.shape[0] - 1
    if num_groups < 0:
        raise ValueError("group_starts needs at least one entry")
    (p_out, p_q, p_k, p_v, p_bt, p_ctx, s, h, d, bs, nb, mb, _mcl, scale_f, dt, part, p_ws,
     ws_bytes, strm) = args
    _check(lib.pa_decode_shared_prefix(p_out, p_q, p_k, p_v, p_bt, p_ctx, _ptr(group_starts),
                                       _ptr(prefix_lens), s, h, d, bs, nb, mb, num_groups,
                                       int(max_group_size), int(max_prefix_len),
                                       int(max_suffix_len), scale_f, dt,
                                       part, int(prefix_partition_size), p_ws, ws_bytes,
                                       _stream(stream, dev) if stream is not None else strm))
    return out


# ----------------------------------------------------------------------------------
# block swap between the GPU pool and a pinned host pool
# ----------------------------------------------------------------------------------

def pa_swap_blocks(dst_key, dst_value, src_key, src_value, block_pairs, stream=None):
    """dst[pair[1]] = src[pair[0]] for K and V, pools in device or pinned host memory
    (see include/pa.h); ``block_pairs`` int32 [n, 2] on the GPU or pinned."""
    _int32(block_pairs)
    if not (dst_key.dtype == dst_value.dtype == src_key.dtype == src_value.dtype):
        raise ValueError("pools must share one dtype")
    nb_d, h, bs, d = dst_key.shape
    nb_s = src_key.shape[0]
    if src_key.shape[1:] != dst_key.shape[1:] or src_value.shape != src_key.shape or \
            dst_value.shape != dst_key.shape:
        raise ValueError("pools must be [num_blocks, H, bs, D] with equal H, bs, D")
    if block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [n, 2]")
    gpu = next((t.device for t in (dst_key, src_key, block_pairs) if t.device.type == "cuda"),
               torch.device("cuda", torch.cuda.current_device()))
    _check(lib.pa_swap_blocks(_ptr(dst_key), _ptr(dst_value), _ptr(src_key), _ptr(src_value),
                              _ptr(block_pairs), block_pairs.shape[0], h, d, bs, nb_s, nb_d,
                              _dtype(dst_key), _stream(stream, gpu)))
