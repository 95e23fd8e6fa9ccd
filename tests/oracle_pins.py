"""Pins for the CPU oracle: checks against facts the pages and the mathematics fix.

Each pin takes the decode function under test, so the same pins run against the
oracle (they must pass) and against copies of it with a planted mistake (each
mistake must trip at least one pin).  Pins never call the oracle function they
check to compute an expected value.

decode_fn signature: decode_fn(q, k_pool, v_pool, block_tables, context_lens, scale)
-> float64 [S, H, D].
"""

from __future__ import annotations

import json
import math
import pathlib

import numpy as np

GOLDEN = pathlib.Path(__file__).resolve().parent / "golden"


def load_block_table_example():
    with open(GOLDEN / "block_table_example.json") as f:
        return json.load(f)


def fixture_pool(num_heads=2, head_dim=4, num_blocks=16):
    """Pool laid out from the block-table sketch of "vLLM basics" §2.3.

    seq_1 owns physical blocks [3, 7, 12] and seq_2 owns [5, 9], block size 16.
    Logical token t of a sequence sits in its table's entry t // 16 at offset t % 16
    (blocks fill slot by slot, "Reading the vLLM source" §2.2, append_tokens).
    Head h of token t holds  K = [t, 0, 0, 0] (h = 0) or [0, t, 0, 0] (h = 1)  and
    V = [t, 1, (-1)^t, h].  Every other slot is NaN.
    """
    ex = load_block_table_example()
    bs = ex["block_size"]
    k_pool = np.full((num_blocks, num_heads, bs, head_dim), np.nan, dtype=np.float32)
    v_pool = np.full_like(k_pool, np.nan)
    tables = []
    for name in ("seq_1", "seq_2"):
        blocks = ex["tables"][name]
        t = 0
        for b in blocks:
            for off in range(bs):
                for h in range(num_heads):
                    k = np.zeros(head_dim, dtype=np.float32)
                    k[h] = t
                    v = np.array([t, 1.0, (-1.0) ** t, h], dtype=np.float32)
                    k_pool[b, h, off] = k
                    v_pool[b, h, off] = v
                t += 1
        tables.append(blocks + [blocks[0]] * (3 - len(blocks)))
    return k_pool, v_pool, np.array(tables, dtype=np.int32), bs


def geometric_closed_form(length: int, rate: float) -> np.ndarray:
    """Expected head-0 output when z_t = rate * t + (alternating term).

    Written from the closed form of a softmax over an arithmetic progression of
    scores: weight_t proportional to exp(rate * t)."""
    t = np.arange(length, dtype=np.float64)
    w = np.exp(rate * t - rate * t.max()) if rate >= 0 else np.exp(rate * t)
    w = w / w.sum()
    alt = (-1.0) ** t
    return np.array([(w * t).sum(), 1.0, (w * alt).sum(), 0.0])


def pin_fixture_geometric(decode_fn):
    """Block-table sketch + closed form: q = [c_s, 0, 0.75, 0] on head 0 of sequence s,
    so z_t = scale * c_s * t; out[0] = sum_t t r^t / sum_t r^t with r = exp(scale * c_s).
    Head 1 uses -c_s.  The two sequences use different rates."""
    k_pool, v_pool, tables, _ = fixture_pool()
    scale = 0.5
    cs = (0.375, 0.25)  # one rate per sequence; exactly representable in float32
    for ctx in ([40, 25], [48, 32], [1, 17], [16, 1]):
        q = np.zeros((2, 2, 4), dtype=np.float32)
        for s, c in enumerate(cs):
            q[s, 0, 0] = c
            q[s, 1, 1] = -c
        q[:, 0, 2] = 0.75  # only V carries the alternating column
        out = decode_fn(q, k_pool, v_pool, tables, np.array(ctx, dtype=np.int32), scale)
        for s, c in enumerate(cs):
            exp0 = geometric_closed_form(ctx[s], scale * c)
            np.testing.assert_allclose(out[s, 0], exp0, rtol=0, atol=1e-12)
            exp1 = geometric_closed_form(ctx[s], -scale * c)
            exp1[3] = 1.0
            np.testing.assert_allclose(out[s, 1], exp1, rtol=0, atol=1e-12)


def pin_context_one_returns_v(decode_fn, batch):
    """A single token gets weight e^0 / e^0 = 1: the output is its V row exactly."""
    ctx = np.ones_like(batch.context_lens)
    out = decode_fn(batch.q, batch.k_pool, batch.v_pool, batch.block_tables, ctx,
                    batch.scale)
    for s in range(batch.q.shape[0]):
        b = int(batch.block_tables[s, 0])
        expect = batch.v_pool[b, :, 0, :].astype(np.float64)
        assert np.array_equal(out[s], expect), "context of one must return its V row"


def pin_uniform_query_gives_mean(decode_fn, batch):
    """q = 0 makes every score 0, so the output is the plain mean of the V rows,
    each read at its (block, offset) position from the table."""
    q = np.zeros_like(batch.q)
    out = decode_fn(q, batch.k_pool, batch.v_pool, batch.block_tables,
                    batch.context_lens, batch.scale)
    bs = batch.k_pool.shape[2]
    for s in range(q.shape[0]):
        length = int(batch.context_lens[s])
        rows = [batch.v_pool[batch.block_tables[s, t // bs], :, t % bs, :]
                for t in range(length)]
        expect = np.mean(np.stack(rows).astype(np.float64), axis=0)
        np.testing.assert_allclose(out[s], expect, rtol=0, atol=1e-12)


def pin_stability(decode_fn):
    """Scores of +-1000 stay finite and put all weight on the top token."""
    rng = np.random.default_rng(7)
    bs, h, d = 16, 1, 8
    k_pool = np.zeros((4, h, bs, d), dtype=np.float32)
    v_pool = rng.standard_normal((4, h, bs, d)).astype(np.float32)
    k_pool[..., 0] = np.linspace(-1000, 1000, 4 * bs).reshape(4, 1, bs)
    tables = np.array([[2, 0, 3, 1]], dtype=np.int32)
    q = np.zeros((1, h, d), dtype=np.float32)
    q[0, 0, 0] = 1.0
    ctx = np.array([64], dtype=np.int32)
    out = decode_fn(q, k_pool, v_pool, tables, ctx, 1.0)
    assert np.all(np.isfinite(out))
    # the largest score is the one with the largest k[0] among the 64 live tokens
    best = max(((b, o) for b in (2, 0, 3, 1) for o in range(bs)),
               key=lambda bo: k_pool[bo[0], 0, bo[1], 0])
    np.testing.assert_allclose(out[0, 0], v_pool[best[0], 0, best[1]], rtol=0, atol=1e-12)


def pin_weights_normalised(weights_fn):
    """Softmax weights are positive and sum to one."""
    rng = np.random.default_rng(11)
    for n in (1, 2, 17, 300):
        keys = rng.standard_normal((n, 16))
        q = rng.standard_normal(16)
        w = weights_fn(q, keys, 0.25)
        assert np.all(w > 0)
        assert abs(w.sum() - 1.0) <= 1e-12


def permuted_batch(batch, seed=3):
    """Same sequences with every physical block id renamed by a random permutation:
    pool block b moves to perm[b] and every table entry is renamed the same way."""
    perm = np.random.default_rng(seed).permutation(batch.k_pool.shape[0])
    k_pool = np.empty_like(batch.k_pool)
    v_pool = np.empty_like(batch.v_pool)
    k_pool[perm] = batch.k_pool
    v_pool[perm] = batch.v_pool
    tables = perm[batch.block_tables].astype(np.int32)
    return k_pool, v_pool, tables


def pin_permutation_invariance(decode_fn, batch):
    """Physical blocks may sit anywhere ("Reading the vLLM source" §2.2; "vLLM basics"
    §2.3): renaming them changes nothing."""
    base = decode_fn(batch.q, batch.k_pool, batch.v_pool, batch.block_tables,
                     batch.context_lens, batch.scale)
    k_pool, v_pool, tables = permuted_batch(batch)
    again = decode_fn(batch.q, k_pool, v_pool, tables, batch.context_lens, batch.scale)
    assert np.array_equal(base, again), "block renaming changed the output"


def shared_vs_private(num_heads=2, head_dim=8, bs=16, prefix_blocks=3, seed=5):
    """Two sequences sharing their first ``prefix_blocks`` blocks by reference, and the
    same two sequences with the shared blocks copied into private ones."""
    rng = np.random.default_rng(seed)
    nb = 4 * prefix_blocks + 8
    k_pool = rng.standard_normal((nb, num_heads, bs, head_dim)).astype(np.float32)
    v_pool = rng.standard_normal((nb, num_heads, bs, head_dim)).astype(np.float32)
    shared = list(range(prefix_blocks))
    tail_a, tail_b = nb - 1, nb - 2
    tables_shared = np.array([shared + [tail_a], shared + [tail_b]], dtype=np.int32)
    private = list(range(prefix_blocks, 2 * prefix_blocks))
    k_priv, v_priv = k_pool.copy(), v_pool.copy()
    k_priv[private] = k_pool[shared]
    v_priv[private] = v_pool[shared]
    tables_private = np.array([shared + [tail_a], private + [tail_b]], dtype=np.int32)
    q = rng.standard_normal((2, num_heads, head_dim)).astype(np.float32)
    ctx = np.array([prefix_blocks * bs + 5, prefix_blocks * bs + 9], dtype=np.int32)
    return q, (k_pool, v_pool, tables_shared), (k_priv, v_priv, tables_private), ctx


def pin_sharing(decode_fn):
    """Ref-counted sharing of prefix blocks ("Reading the vLLM source" §2.2) gives the
    same outputs as private copies of those blocks."""
    q, shared, private, ctx = shared_vs_private()
    a = decode_fn(q, shared[0], shared[1], shared[2], ctx, 0.3)
    b = decode_fn(q, private[0], private[1], private[2], ctx, 0.3)
    assert np.array_equal(a, b)


def pin_poisoned_tail_ignored(decode_fn, batch):
    """Tail slots and unused blocks hold NaN; none may reach the output."""
    out = decode_fn(batch.q, batch.k_pool, batch.v_pool, batch.block_tables,
                    batch.context_lens, batch.scale)
    assert np.all(np.isfinite(out))


def pin_against_brute_force(decode_fn, brute_fn, batch):
    a = decode_fn(batch.q, batch.k_pool, batch.v_pool, batch.block_tables,
                  batch.context_lens, batch.scale)
    b = brute_fn(batch.q, batch.k_pool, batch.v_pool, batch.block_tables,
                 batch.context_lens, batch.scale)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def pin_zero_context(decode_fn, batch):
    ctx = batch.context_lens.copy()
    ctx[0] = 0
    out = decode_fn(batch.q, batch.k_pool, batch.v_pool, batch.block_tables, ctx,
                    batch.scale)
    assert np.array_equal(out[0], np.zeros_like(out[0]))


def all_decode_pins(decode_fn, brute_fn, batches):
    """Run every decode pin; raises AssertionError (or any exception) on failure."""
    pin_fixture_geometric(decode_fn)
    pin_stability(decode_fn)
    pin_sharing(decode_fn)
    for batch in batches:
        pin_context_one_returns_v(decode_fn, batch)
        pin_uniform_query_gives_mean(decode_fn, batch)
        pin_permutation_invariance(decode_fn, batch)
        pin_poisoned_tail_ignored(decode_fn, batch)
        pin_zero_context(decode_fn, batch)
        pin_against_brute_force(decode_fn, brute_fn, batch)


def softmax_logistic_closed_form(delta: float) -> float:
    """Weight of the first of two tokens whose scores differ by ``delta`` = z1 - z0."""
    return 1.0 / (1.0 + math.exp(delta))
