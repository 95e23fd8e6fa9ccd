"""The C-ABI library loads, exports every declared symbol, and rejects bad arguments
on the host (no GPU is touched: every call here fails validation before launch)."""

from __future__ import annotations

import ctypes
import pathlib
import re

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]
HEADERS = sorted((ROOT / "include").glob("*.h"))


def declared_functions():
    names = []
    for h in HEADERS:
        text = h.read_text()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(pa_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def ops():
    from paged_kv_cache_414_amd import ops as _ops
    return _ops


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("pa_decode", "pa_cache_append", "pa_block_copy",
                     "pa_decode_workspace_bytes", "pa_last_error", "pa_status_string"):
        assert required in names


def test_library_exports_every_declared_symbol(ops):
    lib = ctypes.CDLL(str(ops.LIB_PATH))
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"


def test_debug_library_exports_every_declared_symbol(ops):
    """libpa_debug.so: the same kernels and entry points, compiled with PA_DEBUG_CHECKS=1."""
    dbg = ctypes.CDLL(str(ops.DEBUG_LIB_PATH))
    for name in declared_functions():
        assert hasattr(dbg, name), f"{name} declared in include/ but not exported by the debug build"
    dbg.pa_debug_checks.restype = ctypes.c_int32
    assert dbg.pa_debug_checks() == 1
    assert ops.lib.pa_debug_checks() == 0


def test_binding_covers_every_declared_symbol(ops):
    assert sorted(ops.SIGNATURES) == declared_functions()


def test_abi_version_and_status_strings(ops):
    assert ops.lib.pa_abi_version() == 2
    assert ops.lib.pa_status_string(0) == b"PA_OK"
    assert ops.lib.pa_status_string(4) == b"PA_ERR_WORKSPACE"
    assert ops.lib.pa_status_string(99) == b"PA_ERR_UNKNOWN"


def test_partition_planning(ops):
    # explicit sizes must be multiples of the block size
    assert ops.pa_decode_partition_size(96, 32, 16, 2048, 256) == 256
    with pytest.raises(ops.PagedAttentionError):
        ops.pa_decode_partition_size(96, 32, 16, 2048, 100)
    auto = ops.pa_decode_partition_size(96, 32, 16, 2048, 0)
    assert auto > 0 and auto % 16 == 0
    assert ops.pa_decode_num_partitions(8, 32, 32, 32768, 512) == 64
    assert ops.pa_decode_num_partitions(8, 32, 32, 0, 512) == 1
    # one partition needs no workspace; several need m, l (S*H*NP floats each, padded
    # to 256 bytes) and o (S*H*NP*D floats)
    assert ops.pa_decode_workspace_bytes(4, 4, 64, 16, 64, 512) == 0
    s, h, d, np_ = 8, 32, 128, 64
    ml = -(-(s * h * np_ * 4) // 256) * 256
    assert ops.pa_decode_workspace_bytes(s, h, d, 32, 32768, 512) == 2 * ml + s * h * np_ * d * 4


def _bad_decode(ops, **over):
    args = dict(out=1 << 20, q=1 << 20, k=1 << 20, v=1 << 20, bt=1 << 20, ctx=1 << 20,
                S=4, H=4, D=64, bs=16, NB=64, MB=4, maxctx=64, scale=0.125, dtype=0,
                P=0, ws=None, wsb=0)
    args.update(over)
    return ops.lib.pa_decode(args["out"], args["q"], args["k"], args["v"], args["bt"],
                             args["ctx"], args["S"], args["H"], args["D"], args["bs"],
                             args["NB"], args["MB"], args["maxctx"], args["scale"],
                             args["dtype"], args["P"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize("over,status", [
    (dict(D=72), 3),
    (dict(D=512), 3),
    (dict(bs=12), 3),
    (dict(bs=512), 3),
    (dict(dtype=7), 3),
    (dict(maxctx=65), 2),          # more than max_blocks_per_seq * block_size
    (dict(NB=0), 2),
    (dict(H=0), 2),
    (dict(S=70000), 2),
    (dict(P=24), 2),               # not a multiple of the block size
    (dict(scale=float("nan")), 2),
    (dict(q=None), 1),
    (dict(out=(1 << 20) + 4), 2),  # misaligned
    (dict(maxctx=64, P=16), 4),    # four partitions need a workspace
])
def test_decode_rejects_bad_arguments(ops, over, status):
    assert _bad_decode(ops, **over) == status
    assert ops.lib.pa_last_error() != b""


def test_decode_empty_batch_is_a_no_op(ops):
    assert _bad_decode(ops, S=0, out=None, q=None, k=None, v=None, bt=None, ctx=None) == 0
    assert ops.lib.pa_last_error() == b""


def _bad_decode_append(ops, **over):
    args = dict(out=1 << 20, q=1 << 20, k=1 << 20, v=1 << 20, nk=1 << 20, nv=1 << 20, bt=1 << 20,
                ctx=1 << 20, S=4, H=4, D=64, bs=16, NB=64, MB=4, maxctx=64, scale=0.125, dtype=0,
                P=0, ws=None, wsb=0)
    args.update(over)
    return ops.lib.pa_decode_append(args["out"], args["q"], args["k"], args["v"], args["nk"],
                                    args["nv"], args["bt"], args["ctx"], args["S"], args["H"],
                                    args["D"], args["bs"], args["NB"], args["MB"], args["maxctx"],
                                    args["scale"], args["dtype"], args["P"], args["ws"],
                                    args["wsb"], None)


@pytest.mark.parametrize("over,status", [
    (dict(D=72), 3),
    (dict(maxctx=65), 2),
    (dict(P=24), 2),
    (dict(q=None), 1),
    (dict(nk=None), 1),
    (dict(nv=None), 1),
    (dict(nk=(1 << 20) + 8), 2),   # misaligned new rows
    (dict(maxctx=64, P=16), 4),
    (dict(S=65535, H=1, MB=4), 2),  # the store workgroups take grid z-slices after the sequences
    (dict(S=32768, H=1, MB=4), 2),  # 32,768 sequences + 32,768 store workgroups > 65,535
])
def test_decode_append_rejects_bad_arguments(ops, over, status):
    assert _bad_decode_append(ops, **over) == status
    assert ops.lib.pa_last_error() != b""


def test_decode_append_empty_batch_is_a_no_op(ops):
    assert _bad_decode_append(ops, S=0, out=None, q=None, k=None, v=None, nk=None, nv=None,
                              bt=None, ctx=None) == 0


def test_append_and_copy_reject_bad_arguments(ops):
    lib = ops.lib
    p = 1 << 20
    assert lib.pa_cache_append(p, p, p, p, p, 4, 4, 64, 16, 64, 5, None) == 3
    assert lib.pa_cache_append(p, p, p, None, p, 4, 4, 64, 16, 64, 0, None) == 1
    assert lib.pa_cache_append(p, p, p, p, p, -1, 4, 64, 16, 64, 0, None) == 2
    assert lib.pa_cache_append(None, None, None, None, None, 0, 4, 64, 16, 64, 0, None) == 0
    # heads x 16-byte chunks of a row must fit the launch's int32 row index
    assert lib.pa_cache_append(p, p, p, p, p, 4, 1 << 30, 64, 16, 64, 1, None) == 2
    assert lib.pa_block_copy(p, p, p, 2, 4, 72, 16, 64, 0, None) == 3
    assert lib.pa_block_copy(p, p, p, 2, 4, 64, 24, 64, 0, None) == 3
    assert lib.pa_block_copy(p, None, p, 2, 4, 64, 16, 64, 0, None) == 1
    assert lib.pa_block_copy(None, None, None, 0, 4, 64, 16, 64, 0, None) == 0


def _bad_shared(ops, **over):
    p = 1 << 20
    args = dict(out=p, q=p, k=p, v=p, bt=p, ctx=p, gs=p, pl=p, S=16, H=4, D=128, bs=16, NB=64,
                MB=8, G=2, maxg=8, maxp=64, maxs=64, scale=0.125, dtype=1, P=0, Pp=0, ws=p,
                wsb=1 << 30)
    args.update(over)
    return ops.lib.pa_decode_shared_prefix(
        args["out"], args["q"], args["k"], args["v"], args["bt"], args["ctx"], args["gs"],
        args["pl"], args["S"], args["H"], args["D"], args["bs"], args["NB"], args["MB"],
        args["G"], args["maxg"], args["maxp"], args["maxs"], args["scale"], args["dtype"],
        args["P"], args["Pp"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize("over,status", [
    (dict(dtype=0), 3),            # fp32 is not built for the shared-prefix decode
    (dict(bs=4), 3),
    (dict(D=72), 3),
    (dict(maxp=40), 2),            # not a whole number of blocks
    (dict(maxp=-16), 2),
    (dict(maxs=-1), 2),
    (dict(maxp=144), 2),           # more than max_blocks_per_seq * block_size
    (dict(maxs=129), 2),
    (dict(Pp=24), 2),              # prefix partitions are whole 16-token tiles
    (dict(P=24), 2),
    (dict(G=-1), 2),
    (dict(maxg=-1), 2),
    (dict(scale=float("inf")), 2),
    (dict(pl=None), 1),
    (dict(gs=None), 1),
    (dict(ws=None), 4),
    (dict(wsb=16), 4),
])
def test_shared_prefix_rejects_bad_arguments(ops, over, status):
    assert _bad_shared(ops, **over) == status
    assert ops.lib.pa_last_error() != b""


def test_decode_workgroup_size_policy(ops):
    import torch
    # 16 waves: partitions of 32+ units and 1024+ workgroups; else 8
    assert ops.pa_decode_waves(96, 32, 128, 16, 2036) == 16     # 3,072 x 128 units
    assert ops.pa_decode_waves(16, 32, 128, 16, 8192) == 8      # 512 workgroups
    assert ops.pa_decode_waves(64, 32, 128, 16, 300) == 8       # 19 units per partition
    assert ops.pa_decode_waves(64, 32, 128, 16, 562) == 16      # 36 units, 2,048 workgroups
    assert ops.pa_decode_waves(64, 32, 128, 16, 562, 256) == 8  # 16 units per partition
    # units of 8 tokens (block size 8, fp32 D64: 4 rows per load, 8 loads would be 32 tokens)
    assert ops.pa_decode_waves(64, 16, 64, 8, 600, 0, torch.float32) == 16
    # blocks of 256 tokens are walked in units of 32 (fp16 D128: 4 rows per load x 8 loads)
    assert ops.pa_decode_waves(96, 32, 128, 256, 700) == 8      # P 768: 24 units
    assert ops.pa_decode_waves(96, 32, 128, 256, 1000) == 16    # P 1024: 32 units
    with pytest.raises(ops.PagedAttentionError):
        ops.pa_decode_waves(96, 32, 72, 16, 2036)


def test_shared_prefix_planning(ops):
    # an empty batch needs nothing and enqueues nothing
    assert _bad_shared(ops, S=0, out=None, q=None, k=None, v=None, bt=None, ctx=None,
                       gs=None, pl=None, ws=None, wsb=0) == 0
    s, h, d = 64, 32, 128
    n = ops.pa_decode_shared_prefix_workspace_bytes(s, h, d, 16, 8, 1024, 272, 0, 256)
    # 4 prefix partitions of 256 tokens + 1 partition for the 272 tokens after them
    slots = 4 + ops.pa_decode_num_partitions(s, h, 16, 272, 0)
    ml = -(-(s * h * slots * 4) // 256) * 256
    assert n == 2 * ml + s * h * slots * d * 4

    def prefix_slots(groups, max_group_size, maxp):
        # S*H*4 is a multiple of 256 here, so the bytes are slots x S*H*(D+2)*4 exactly
        n = ops.pa_decode_shared_prefix_workspace_bytes(s, h, d, 16, groups, maxp, 16, 0, 0,
                                                        max_group_size)
        return n // (s * h * (d + 2) * 4) - ops.pa_decode_num_partitions(s, h, 16, 16, 0)
    # the library's prefix partition: the whole prefix while (groups x 16-member tiles
    # x heads) fills 256 workgroups, halved otherwise (not below 64 tokens)
    assert prefix_slots(8, 8, 1024) == 1        # 8 x 1 x 32 = 256 workgroups
    assert prefix_slots(1, 8, 1024) == 8        # 32 per partition: 8 partitions of 128
    assert prefix_slots(1, 64, 1024) == 2       # 4 tiles x 32 = 128: 2 partitions of 512
    assert prefix_slots(1, 0, 1024) == 2        # 0: the average group (64 members) decides
    assert prefix_slots(2, 0, 1024) == 2        # average 32 members: 2 x 2 x 32 = 128
    assert prefix_slots(1, 128, 512) == 1       # 8 tiles x 32 = 256 already
    # head dims 64, 80, 96, 128 and 256 are built for the shared-prefix decode; others are refused
    for dd in (64, 80, 96, 256):
        assert ops.pa_decode_shared_prefix_workspace_bytes(s, h, dd, 16, 8, 1024, 272) > 0
    for dd in (72, 112):
        assert ops.lib.pa_decode_shared_prefix_workspace_bytes(s, h, dd, 16, 8, 0, 1024, 272, 0, 0) == 0
        assert b"head_dim" in ops.lib.pa_last_error()
    # blocks of 8 tokens: the pass after the prefix is planned for 8 more tokens (a prefix
    # may end half a 16-token tile past the prefix pass's last whole tile)
    n8 = ops.pa_decode_shared_prefix_workspace_bytes(s, h, d, 8, 8, 1024, 256, 256, 256)
    slots8 = 4 + ops.pa_decode_num_partitions(s, h, 8, 264, 256)
    assert slots8 == 6
    ml8 = -(-(s * h * slots8 * 4) // 256) * 256
    assert n8 == 2 * ml8 + s * h * slots8 * d * 4
    assert ops.lib.pa_decode_shared_prefix_workspace_bytes(s, h, d, 4, 8, 0, 1024, 272, 0, 0) == 0
    # a prefix that is not a whole number of blocks is refused
    assert ops.lib.pa_decode_shared_prefix_workspace_bytes(s, h, d, 16, 8, 0, 1000, 272, 0, 0) == 0
    assert ops.lib.pa_last_error() != b""
    with pytest.raises(ops.PagedAttentionError):
        ops.pa_decode_shared_prefix_workspace_bytes(s, h, d, 16, 8, 1000, 272)


def test_swap_rejects_bad_arguments(ops):
    lib = ops.lib
    p = 1 << 20
    # dtype, shape, sizes and NULLs are checked before any pointer is looked up
    assert lib.pa_swap_blocks(p, p, p, p, p, 2, 4, 64, 16, 8, 8, 5, None) == 3
    assert lib.pa_swap_blocks(p, p, p, p, p, 2, 4, 72, 16, 8, 8, 0, None) == 3
    assert lib.pa_swap_blocks(p, p, p, p, p, -1, 4, 64, 16, 8, 8, 0, None) == 2
    assert lib.pa_swap_blocks(p, p, p, p, p, 2, 4, 64, 16, 0, 8, 0, None) == 2
    assert lib.pa_swap_blocks(p, None, p, p, p, 2, 4, 64, 16, 8, 8, 0, None) == 1
    assert lib.pa_swap_blocks(p + 4, p, p, p, p, 2, 4, 64, 16, 8, 8, 0, None) == 2
    assert lib.pa_swap_blocks(None, None, None, None, None, 0, 4, 64, 16, 8, 8, 0, None) == 0


def test_last_error_is_per_thread(ops):
    """Threads failing at once each read back their own message (pa_last_error is
    thread-local; ctypes releases the GIL around the calls)."""
    import threading
    dims = [72, 88, 104, 120, 136, 152, 168, 184]
    bad = []

    def worker(d):
        for _ in range(400):
            st = _bad_decode(ops, D=d)
            msg = ops.lib.pa_last_error().decode()
            if st != 3 or f"head_dim {d} " not in msg:
                bad.append((d, st, msg))
                return

    threads = [threading.Thread(target=worker, args=(d,)) for d in dims]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not bad, bad[:3]


def test_noalloc_scratch_size_and_host_checks(ops):
    """pa_decode_noalloc: the binding's scratch size is the header's; invalid arguments
    are refused by pa_decode's checks and oversize requests by the size check, both
    before anything touches a GPU."""
    text = (ROOT / "include" / "pa.h").read_text()
    m = re.search(r"#define PA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == ops.PA_NOALLOC_SCRATCH_BYTES
    fake = 1 << 20
    lib = ops.lib
    assert lib.pa_decode_noalloc(fake, fake, fake, fake, fake, fake, 4, 4, 72, 16, 64, 4, 64,
                                 0.125, ops.PA_F32, 0, None) == 3
    assert lib.pa_decode_noalloc(fake, None, fake, fake, fake, fake, 4, 4, 64, 16, 64, 4, 64,
                                 0.125, ops.PA_F32, 0, None) == 1
    s, h, d, bs, mcl, part = 4096, 32, 128, 16, 8192, 512
    assert lib.pa_decode_noalloc(fake, fake, fake, fake, fake, fake, s, h, d, bs, 100000,
                                 mcl // bs, mcl, 0.1, ops.PA_F16, part, None) == 4
    assert b"scratch" in lib.pa_last_error()
    assert lib.pa_decode_noalloc(None, None, None, None, None, None, 0, 4, 64, 16, 64, 4, 64,
                                 0.125, ops.PA_F32, 0, None) == 0


def test_decode_hints_are_checked_on_the_host(ops):
    """pa_decode_ex / pa_decode_append_ex: a workgroup size other than 0, 8 or 16 and a
    misaligned order are refused before launch; NULL hints behave as the plain call."""
    fake = 1 << 20
    lib = ops.lib
    base = (fake, fake, fake, fake, fake, fake, 4, 4, 64, 16, 64, 4, 64, 0.125, ops.PA_F32, 0,
            None, 0)
    for waves, order, status in ((12, None, 2), (8, fake + 2, 2)):
        h = ops.DecodeHints(order, waves)
        assert lib.pa_decode_ex(*base, ctypes.byref(h), None) == status
        assert b"hints" in lib.pa_last_error()
        assert lib.pa_decode_append_ex(*base[:4], fake, fake, *base[4:], ctypes.byref(h),
                                       None) == status
    # NULL hints and an empty batch: nothing to do
    empty = (None,) * 6 + (0,) + base[7:]
    assert lib.pa_decode_ex(*empty, None, None) == 0
