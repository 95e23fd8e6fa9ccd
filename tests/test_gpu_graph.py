"""The append + decode step recorded as a HIP graph and replayed.

Each replay is checked against the same step launched eagerly on a second copy of
the pool (bit for bit: same kernels, same grid bound) and against the CPU oracle
(2e-3), with eager work and synchronisation between replays.  Contexts grow by one
token per replay and one sequence is retired (context 0, slot -1) mid-way.  The
graph records either the two launches (pa_cache_append, pa_decode) or the single
pa_decode_append; the eager reference is always the two launches."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_414_amd import blocks, workloads
from tests.gpu_util import dev, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("fused", [False, True], ids=["two_launches", "fused"])
@pytest.mark.parametrize("partition", [0, 64])
def test_graph_replays_match_eager_and_oracle(partition, fused):
    from paged_kv_cache_414_amd import graphs, ops
    b = workloads.make_static_batch("graph", seed=19, num_seqs=6, num_heads=4, head_dim=128,
                                    block_size=16, ctx_low=1, ctx_high=300, dtype=np.float16,
                                    pool_slack=1.5, max_blocks_per_seq=24)
    bound = 24 * 16
    k_host, v_host = b.k_pool.copy(), b.v_pool.copy()
    k_a, v_a = dev(b.k_pool), dev(b.v_pool)  # stepped by the graph
    k_b, v_b = dev(b.k_pool), dev(b.v_pool)  # stepped eagerly
    note(f"capture DecodeStepGraph P={partition} fused={fused}")
    g = graphs.DecodeStepGraph(k_a, v_a, b.num_seqs, 24, bound, b.scale, partition, fused=fused)
    out_b = torch.empty_like(g.out)
    ws_b = ops.workspace_for(g.q, k_b, bound, partition)

    # spare blocks for sequences that cross a block boundary while stepping
    used = {int(x) for s in range(b.num_seqs) for x in b.block_tables[s, :-(-int(b.context_lens[s]) // 16)]}
    spare = [x for x in range(b.num_blocks) if x not in used]
    tables = b.block_tables.copy()
    ctx = b.context_lens.copy()
    rng = np.random.default_rng(3)
    for r in range(5):
        if r == 3:
            ctx[2] = 0  # sequence 2 finished: no more appends, empty context
        pos = ctx.copy()
        live = ctx > 0 if r >= 3 else np.ones_like(ctx, dtype=bool)
        for s in range(b.num_seqs):
            if live[s] and pos[s] % 16 == 0:
                tables[s, pos[s] // 16] = spare.pop()
        slots = np.where(live, blocks.slots_for_positions(tables, pos, 16), -1).astype(np.int32)
        ctx = np.where(live, ctx + 1, 0).astype(np.int32)
        q = workloads.normal(rng, b.q.shape, np.float16)
        nk = workloads.normal(rng, b.q.shape, np.float16)
        nv = workloads.normal(rng, b.q.shape, np.float16)
        for t, a in ((g.q, q), (g.new_k, nk), (g.new_v, nv), (g.slots, slots),
                     (g.block_tables, tables), (g.context_lens, ctx)):
            t.copy_(torch.from_numpy(np.ascontiguousarray(a)))
        note(f"graph replay {r}")
        g.replay()
        # the same step, eagerly, on the second pool
        ops.pa_cache_append(k_b, v_b, dev(nk), dev(nv), dev(slots))
        ops.pa_decode(out_b, dev(q), k_b, v_b, dev(tables), dev(ctx), b.scale, bound, partition,
                      ws_b)
        torch.cuda.synchronize()
        got, eager = g.out.cpu().numpy(), out_b.cpu().numpy()
        assert np.array_equal(got.view(np.uint16), eager.view(np.uint16)), r
        oracle.cache_append(k_host, v_host, nk, nv, slots, inplace=True)
        want = oracle.decode(q, k_host, v_host, tables, ctx, b.scale)
        assert float(np.max(np.abs(got.astype(np.float64) - want))) <= 2e-3, r
        assert np.array_equal(k_a.cpu().numpy().view(np.uint16), k_host.view(np.uint16)), r
        assert np.array_equal(got[2] == 0, np.ones_like(got[2], dtype=bool)) or r < 3
