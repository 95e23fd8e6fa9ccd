"""The CPU oracle against its pins, and planted mistakes against the same pins.

A planted mistake is a copy of the oracle's decode with one plausible error (dropped
scale, wrong sign, swapped block/offset, off-by-one length, wrong head, transposed
operand, ...).  Each must trip at least one pin, which shows the pins can tell a
correct oracle from a subtly wrong one.
"""

from __future__ import annotations

import json

import numpy as np
import pytest

import oracle
from paged_kv_cache_414_amd import workloads
from tests import oracle_pins as pins


@pytest.fixture(scope="module")
def tiny_batches():
    return [workloads.tiny_fp32(seed=1), workloads.tiny_fp32(seed=101)]


def oracle_decode(q, k, v, t, c, s):
    return oracle.decode(q, k, v, t, c, s)


def oracle_decode_slow(q, k, v, t, c, s):
    return oracle.decode(q, k, v, t, c, s, fast=False)


# ----------------------------------------------------------------------------------
# the oracle passes every pin
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("fn", [oracle_decode, oracle_decode_slow], ids=["fast", "slow"])
def test_oracle_passes_all_decode_pins(fn, tiny_batches):
    pins.all_decode_pins(fn, oracle.brute_force_decode, tiny_batches)


def test_weights_normalised():
    pins.pin_weights_normalised(oracle.attention_weights)


def test_two_token_logistic():
    """Two tokens whose scores differ by delta: weight of the first is 1/(1+e^delta)."""
    keys = np.array([[1.0, 0.0], [3.0, 0.0]])
    q = np.array([0.4, 9.0])
    w = oracle.attention_weights(q, keys, 0.5)
    delta = 0.5 * (3.0 - 1.0) * 0.4
    assert abs(w[0] - pins.softmax_logistic_closed_form(delta)) < 1e-15


def test_brute_force_matches_on_larger_tiny_seeds():
    for seed in (2, 3, 102):
        b = workloads.tiny_fp32(seed=seed)
        pins.pin_against_brute_force(oracle_decode, oracle.brute_force_decode, b)


def _split_points(length, cuts):
    pts = sorted({0, length, *[c for c in cuts if 0 < c < length]})
    return list(zip(pts[:-1], pts[1:]))


def _pin_lse_merge(state_fn, merge_fn, batches):
    """Merging partition states by log-sum-exp gives back the unsplit attention
    (the brute-force scalar decode, not the oracle's own decode)."""
    for batch in batches:
        full = oracle.brute_force_decode(batch.q, batch.k_pool, batch.v_pool,
                                         batch.block_tables, batch.context_lens, batch.scale)
        for s in range(batch.num_seqs):
            length = int(batch.context_lens[s])
            for cuts in ([16], [7, 33], [1, 2, 3, 40], list(range(16, 64, 16))):
                parts = _split_points(length, cuts)
                for h in range(batch.num_heads):
                    st = [state_fn(batch.q[s, h], batch.k_pool, batch.v_pool,
                                   batch.block_tables[s], length, h, batch.scale, a, b)
                          for a, b in parts]
                    merged = merge_fn(*zip(*st))
                    np.testing.assert_allclose(merged, full[s, h], rtol=0, atol=1e-12)


def test_lse_merge_equals_unsplit(tiny_batches):
    _pin_lse_merge(oracle.partition_state, oracle.merge_partition_states, tiny_batches)


def _merge_without_rescaled_sums(ms, ls, os_):
    ms, ls, os_ = (np.asarray(x, dtype=np.float64) for x in (ms, ls, os_))
    f = np.exp(ms - ms.max())
    return (f[:, None] * os_).sum(axis=0) / ls.sum()


def _merge_by_averaging(ms, ls, os_):
    os_ = np.asarray(os_, dtype=np.float64)
    return (os_ / np.asarray(ls, dtype=np.float64)[:, None]).mean(axis=0)


def _merge_wrong_sign(ms, ls, os_):
    ms, ls, os_ = (np.asarray(x, dtype=np.float64) for x in (ms, ls, os_))
    f = np.exp(ms.max() - ms)
    return (f[:, None] * os_).sum(axis=0) / (f * ls).sum()


def _state_skipping_first_token(q_row, k_pool, v_pool, row, length, head, scale, start, stop):
    if min(stop, length) - start > 1:
        start += 1
    return oracle.partition_state(q_row, k_pool, v_pool, row, length, head, scale, start, stop)


@pytest.mark.parametrize("state_fn, merge_fn", [
    (oracle.partition_state, _merge_without_rescaled_sums),
    (oracle.partition_state, _merge_by_averaging),
    (oracle.partition_state, _merge_wrong_sign),
    (_state_skipping_first_token, oracle.merge_partition_states),
], ids=["unscaled-sums", "average", "wrong-sign", "skip-first-token"])
def test_planted_merge_mistake_is_caught(state_fn, merge_fn, tiny_batches):
    with pytest.raises(AssertionError):
        _pin_lse_merge(state_fn, merge_fn, tiny_batches[:1])


def test_partition_state_definition():
    """A single-token partition has m = z, l = 1 and o = its V row."""
    b = workloads.tiny_fp32(seed=4)
    s, h = 0, 1
    blk = int(b.block_tables[s, 0])
    m, l, o = oracle.partition_state(b.q[s, h], b.k_pool, b.v_pool, b.block_tables[s],
                                     b.context_lens[s], h, b.scale, 0, 1)
    z = b.scale * float(np.dot(b.q[s, h].astype(np.float64),
                               b.k_pool[blk, h, 0].astype(np.float64)))
    assert abs(m - z) < 1e-12 and l == 1.0
    assert np.array_equal(o, b.v_pool[blk, h, 0].astype(np.float64))


# ----------------------------------------------------------------------------------
# append / block copy / slot addressing against the block-table sketch
# ----------------------------------------------------------------------------------

def test_slot_of_block_table_example():
    """seq_1 -> physical blocks [3, 7, 12], block size 16 ("vLLM basics" §2.3):
    position 0 -> block 3 offset 0 = slot 48; position 17 -> block 7 offset 1 = slot
    113; position 39 -> block 12 offset 7 = slot 199; seq_2 -> [5, 9]: position 31 ->
    block 9 offset 15 = slot 159."""
    ex = pins.load_block_table_example()
    t1, t2 = ex["tables"]["seq_1"], ex["tables"]["seq_2"]
    assert oracle.slot_of(t1, 0, 16) == 48
    assert oracle.slot_of(t1, 17, 16) == 113
    assert oracle.slot_of(t1, 39, 16) == 199
    assert oracle.slot_of(t2, 31, 16) == 159
    assert oracle.token_location(t2, 16, 16) == (9, 0)


def test_slots_for_positions_block_table_example():
    """The batch form the step replays use, on the same sketch stacked into one
    [2, 3] table (seq_2's unused third entry padded with a value no slot may come
    from): (seq_1, 0) -> 48, (seq_1, 17) -> 113, (seq_1, 39) -> 199, (seq_2, 31) ->
    159, (seq_2, 16) -> block 9 offset 0 = 144, (seq_2, 0) -> block 5 offset 0 = 80."""
    ex = pins.load_block_table_example()
    t1, t2 = ex["tables"]["seq_1"], ex["tables"]["seq_2"]
    tables = np.array([t1, t2 + [-1000]], dtype=np.int32)
    got = oracle.slots_for_positions(tables, [0, 0, 0, 1, 1, 1], [0, 17, 39, 31, 16, 0],
                                     ex["block_size"])
    assert got.tolist() == [48, 113, 199, 159, 144, 80]
    # the sequence index selects the row: the same positions on the other row differ
    swapped = oracle.slots_for_positions(tables, [1, 1], [0, 17], ex["block_size"])
    assert swapped.tolist() == [80, 145]


def _append_case():
    rng = np.random.default_rng(0)
    k = rng.standard_normal((16, 2, 16, 4)).astype(np.float16)
    v = rng.standard_normal((16, 2, 16, 4)).astype(np.float16)
    key = rng.standard_normal((3, 2, 4)).astype(np.float16)
    value = rng.standard_normal((3, 2, 4)).astype(np.float16)
    return k, v, key, value


def check_append(append_fn):
    k, v, key, value = _append_case()
    slots = np.array([113, -1, 48], dtype=np.int32)  # block 7 off 1; skipped; block 3 off 0
    k2, v2 = append_fn(k, v, key, value, slots)
    ek, ev = k.copy(), v.copy()
    ek[7, :, 1, :], ev[7, :, 1, :] = key[0], value[0]
    ek[3, :, 0, :], ev[3, :, 0, :] = key[2], value[2]
    assert np.array_equal(k2.view(np.uint16), ek.view(np.uint16))
    assert np.array_equal(v2.view(np.uint16), ev.view(np.uint16))


def test_cache_append_fixture():
    check_append(oracle.cache_append)


def test_cache_append_rejects_repeated_slot():
    k, v, key, value = _append_case()
    with pytest.raises(ValueError):
        oracle.cache_append(k, v, key, value, np.array([5, 5, -1]))


def check_block_copy(copy_fn):
    k, v, _, _ = _append_case()
    k2, v2 = copy_fn(k, v, np.array([[3, 10], [5, 11]], dtype=np.int32))
    ek, ev = k.copy(), v.copy()
    ek[10], ek[11] = k[3], k[5]
    ev[10], ev[11] = v[3], v[5]
    assert np.array_equal(k2.view(np.uint16), ek.view(np.uint16))
    assert np.array_equal(v2.view(np.uint16), ev.view(np.uint16))


def test_block_copy_fixture():
    check_block_copy(oracle.block_copy)


def test_block_copy_preconditions():
    k, v, _, _ = _append_case()
    with pytest.raises(ValueError):
        oracle.block_copy(k, v, [[1, 2], [3, 2]])
    with pytest.raises(ValueError):
        oracle.block_copy(k, v, [[1, 2], [2, 4]])


def test_golden_kv_bytes_arithmetic_is_consistent():
    """The page's byte figures are products of their factors (guards the fixture)."""
    with open(pins.GOLDEN / "kv_bytes.json") as f:
        cases = json.load(f)["cases"]
    for c in cases:
        prod = (2 * c["layers"] * c["heads"] * c["head_dim"] * c["bytes_per_elem"]
                * c["tokens"] * c["seqs"])
        assert prod == c["bytes"]
        assert abs(c["bytes"] / 2**30 - c["quoted_gb"]) < 0.1 * c["quoted_gb"] + 0.05


# ----------------------------------------------------------------------------------
# planted mistakes
# ----------------------------------------------------------------------------------

def _mutant(score=None, gather=None, norm=None, length=None, head=None, qsel=None,
            keys_from_v=False, out_from_k=False, no_max=False):
    """A copy of the oracle's decode with one step replaced."""

    def gather_ok(pool, row, n, h):
        bs = pool.shape[2]
        rows = []
        for t in range(n):
            rows.append(pool[row[t // bs], h, t % bs, :])
        return np.array(rows, dtype=np.float64).reshape(n, pool.shape[3])

    g = gather or gather_ok

    def fn(q, k_pool, v_pool, tables, ctx, scale):
        s_count, h_count, d = q.shape
        out = np.zeros((s_count, h_count, d))
        for s in range(s_count):
            n = int(ctx[s]) if length is None else length(int(ctx[s]))
            if int(ctx[s]) == 0:
                continue
            for h in range(h_count):
                hh = h if head is None else head(h, h_count)
                ss = s if qsel is None else qsel(s, s_count)
                keys = g(v_pool if keys_from_v else k_pool, tables[s], n, hh)
                vals = g(k_pool if out_from_k else v_pool, tables[s], n, hh)
                z = keys @ q[ss, h].astype(np.float64)
                z = scale * z if score is None else score(z, scale)
                e = np.exp(z) if no_max else np.exp(z - z.max())
                w = e / e.sum() if norm is None else norm(e)
                out[s, h] = w @ vals
        return out

    return fn


def _gather_swapped(pool, row, n, h):
    bs = pool.shape[2]
    return np.array([pool[row[t % bs], h, t // bs, :] for t in range(n)],
                    dtype=np.float64).reshape(n, pool.shape[3])


def _gather_axes_transposed(pool, row, n, h):
    bs = pool.shape[2]
    return np.array([pool[row[t // bs], t % bs, h, :] for t in range(n)],
                    dtype=np.float64).reshape(n, pool.shape[3])


def _gather_reversed_blocks(pool, row, n, h):
    bs = pool.shape[2]
    nb = -(-n // bs)
    return np.array([pool[row[nb - 1 - t // bs], h, t % bs, :] for t in range(n)],
                    dtype=np.float64).reshape(n, pool.shape[3])


MUTANTS = {
    "dropped_scale": _mutant(score=lambda z, s: z),
    "negated_scores": _mutant(score=lambda z, s: -s * z),
    "scale_squared": _mutant(score=lambda z, s: s * s * z),
    "swapped_block_offset": _mutant(gather=_gather_swapped),
    "pool_axes_transposed": _mutant(gather=_gather_axes_transposed),
    "reversed_block_order": _mutant(gather=_gather_reversed_blocks),
    "context_minus_one": _mutant(length=lambda n: max(n - 1, 1)),
    "context_plus_one": _mutant(length=lambda n: n + 1),
    "no_max_subtraction": _mutant(no_max=True),
    "wrong_head": _mutant(head=lambda h, n: (h + 1) % n),
    "wrong_sequence_query": _mutant(qsel=lambda s, n: (s + 1) % n),
    "keys_from_value_pool": _mutant(keys_from_v=True),
    "output_from_key_pool": _mutant(out_from_k=True),
    "normalise_by_count": _mutant(norm=lambda e: e / e.size),
}


def test_correct_copy_of_decode_passes(tiny_batches):
    """The mutant scaffolding itself, with no mistake planted, passes every pin."""
    pins.all_decode_pins(_mutant(), oracle.brute_force_decode, tiny_batches)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tiny_batches):
    fn = MUTANTS[name]
    with np.errstate(all="ignore"):
        with pytest.raises(Exception):
            pins.all_decode_pins(fn, oracle.brute_force_decode, tiny_batches)


def _append_swapped(k_pool, v_pool, key, value, slots):
    bs = k_pool.shape[2]
    k2, v2 = k_pool.copy(), v_pool.copy()
    for i, s in enumerate(slots):
        if s < 0:
            continue
        o, b = divmod(int(s), bs)
        k2[b, :, o, :], v2[b, :, o, :] = key[i], value[i]
    return k2, v2


def _append_key_twice(k_pool, v_pool, key, value, slots):
    return oracle.cache_append(k_pool, v_pool, key, key, slots)


def _copy_k_only(k_pool, v_pool, pairs):
    k2, _ = oracle.block_copy(k_pool, v_pool, pairs)
    return k2, v_pool.copy()


@pytest.mark.parametrize("fn", [_append_swapped, _append_key_twice])
def test_planted_append_mistake_is_caught(fn):
    with pytest.raises(Exception):
        check_append(fn)


def test_planted_copy_mistake_is_caught():
    with pytest.raises(Exception):
        check_block_copy(_copy_k_only)


# ----------------------------------------------------------------------------------
# swapping blocks between two pools ("Reading the vLLM source" §3)
# ----------------------------------------------------------------------------------

def _labelled_pool(num_blocks, offset):
    """Pools whose every element names its block: K = offset + id, V = -(offset + id)."""
    ids = np.arange(num_blocks, dtype=np.float32)[:, None, None, None] + offset
    k = np.broadcast_to(ids, (num_blocks, 2, 4, 8)).astype(np.float32).copy()
    return k, -k


def check_swap(swap_fn):
    """Device pool of 12 blocks (labels 0..11), host pool of 6 (labels 100..105):
    swapping out (src in the device pool, dst in the host pool) leaves host block dst
    labelled with device id src, everything else untouched; swapping back in restores
    the device pool."""
    dk, dv = _labelled_pool(12, 0.0)
    hk, hv = _labelled_pool(6, 100.0)
    out_pairs = np.array([[7, 0], [2, 5], [11, 3]], dtype=np.int32)
    hk2, hv2 = swap_fn(hk, hv, dk, dv, out_pairs)
    want = {0: 7.0, 5: 2.0, 3: 11.0, 1: 101.0, 2: 102.0, 4: 104.0}
    for blk, label in want.items():
        assert np.all(hk2[blk] == label) and np.all(hv2[blk] == -label), blk
    # the device blocks are reused by someone else, then the data comes back in
    dk_reused, dv_reused = np.zeros_like(dk), np.zeros_like(dv)
    back = out_pairs[:, ::-1].copy()  # (host, device)
    dk3, dv3 = swap_fn(dk_reused, dv_reused, hk2, hv2, back)
    for dev_blk in (7, 2, 11):
        assert np.array_equal(dk3[dev_blk], dk[dev_blk]) and np.array_equal(dv3[dev_blk], dv[dev_blk])
    assert np.all(dk3[[0, 1, 3, 4, 5, 6, 8, 9, 10]] == 0)


def test_swap_blocks_pins():
    check_swap(oracle.swap_blocks)
    with pytest.raises(ValueError):
        oracle.swap_blocks(*_labelled_pool(4, 0.0), *_labelled_pool(4, 9.0), [[0, 1], [2, 1]])


def _swap_reversed(dst_k, dst_v, src_k, src_v, pairs):
    return oracle.swap_blocks(dst_k, dst_v, src_k, src_v, np.asarray(pairs)[:, ::-1])


def _swap_k_only(dst_k, dst_v, src_k, src_v, pairs):
    k, _ = oracle.swap_blocks(dst_k, dst_v, src_k, src_v, pairs)
    return k, dst_v.copy()


@pytest.mark.parametrize("fn", [_swap_reversed, _swap_k_only])
def test_planted_swap_mistake_is_caught(fn):
    with pytest.raises(Exception):
        check_swap(fn)
