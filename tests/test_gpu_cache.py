"""pa_cache_append and pa_block_copy on the GPU: bit-exact against the oracle over
the whole pool (untouched slots included)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_414_amd import workloads
from tests.gpu_util import dev, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bits(a):
    return a.view(np.uint16 if a.dtype == np.float16 else np.uint32)


CASES = [(np.float16, 128, 16, 32), (np.float16, 64, 32, 4), (np.float16, 128, 8, 7),
         (np.float32, 64, 16, 4), (np.float32, 128, 32, 3), (np.float16, 80, 64, 5),
         (np.float16, 256, 256, 2), (np.float32, 96, 128, 3)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{np.dtype(c[0]).name}-D{c[1]}-bs{c[2]}-H{c[3]}")
@pytest.mark.parametrize("num_tokens", [1, 64, 333])
def test_cache_append_bit_exact(case, num_tokens):
    from paged_kv_cache_414_amd import ops
    dtype, d, bs, h = case
    rng = np.random.default_rng(num_tokens * 31 + d + bs)
    nb = 96
    k_pool = workloads.normal(rng, (nb, h, bs, d), dtype)
    v_pool = workloads.normal(rng, (nb, h, bs, d), dtype)
    key = workloads.normal(rng, (num_tokens, h, d), dtype)
    value = workloads.normal(rng, (num_tokens, h, d), dtype)
    slots = rng.choice(nb * bs, size=num_tokens, replace=False).astype(np.int32)
    slots[rng.random(num_tokens) < 0.1] = -1  # some rows are skipped
    kd, vd = dev(k_pool), dev(v_pool)
    note(f"pa_cache_append T={num_tokens} {case}")
    ops.pa_cache_append(kd, vd, dev(key), dev(value), dev(slots))
    torch.cuda.synchronize()
    ek, ev = oracle.cache_append(k_pool, v_pool, key, value, slots)
    assert np.array_equal(_bits(kd.cpu().numpy()), _bits(ek))
    assert np.array_equal(_bits(vd.cpu().numpy()), _bits(ev))


def test_cache_append_more_tokens_than_one_grid_column():
    """70,000 rows: more than the 65,535 tokens one launch column holds, so workgroups
    walk several tokens each."""
    from paged_kv_cache_414_amd import ops
    rng = np.random.default_rng(65536)
    h, bs, d, nb, num_tokens = 2, 16, 64, 5000, 70000
    k_pool = workloads.normal(rng, (nb, h, bs, d), np.float16)
    v_pool = workloads.normal(rng, (nb, h, bs, d), np.float16)
    key = workloads.normal(rng, (num_tokens, h, d), np.float16)
    value = workloads.normal(rng, (num_tokens, h, d), np.float16)
    slots = rng.choice(nb * bs, size=num_tokens, replace=False).astype(np.int32)
    slots[rng.random(num_tokens) < 0.05] = -1
    kd, vd = dev(k_pool), dev(v_pool)
    note(f"pa_cache_append T={num_tokens} H={h} D={d} bs={bs}")
    ops.pa_cache_append(kd, vd, dev(key), dev(value), dev(slots))
    torch.cuda.synchronize()
    ek, ev = oracle.cache_append(k_pool, v_pool, key, value, slots)
    assert np.array_equal(_bits(kd.cpu().numpy()), _bits(ek))
    assert np.array_equal(_bits(vd.cpu().numpy()), _bits(ev))


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{np.dtype(c[0]).name}-D{c[1]}-bs{c[2]}-H{c[3]}")
@pytest.mark.parametrize("num_pairs", [1, 56, 200])
def test_block_copy_bit_exact(case, num_pairs):
    from paged_kv_cache_414_amd import ops
    dtype, d, bs, h = case
    rng = np.random.default_rng(num_pairs * 17 + d + bs)
    nb = 2 * num_pairs + 16
    k_pool = workloads.normal(rng, (nb, h, bs, d), dtype)
    v_pool = workloads.normal(rng, (nb, h, bs, d), dtype)
    perm = rng.permutation(nb)
    dsts = perm[:num_pairs]
    src_pool = perm[num_pairs:]
    srcs = rng.choice(src_pool, size=num_pairs, replace=True)  # a source may serve many
    pairs = np.stack([srcs, dsts], axis=1).astype(np.int32)
    kd, vd = dev(k_pool), dev(v_pool)
    note(f"pa_block_copy n={num_pairs} {case}")
    ops.pa_block_copy(kd, vd, dev(pairs))
    torch.cuda.synchronize()
    ek, ev = oracle.block_copy(k_pool, v_pool, pairs)
    assert np.array_equal(_bits(kd.cpu().numpy()), _bits(ek))
    assert np.array_equal(_bits(vd.cpu().numpy()), _bits(ev))


def test_empty_calls_are_no_ops():
    from paged_kv_cache_414_amd import ops
    k = torch.zeros((4, 2, 16, 64), dtype=torch.float16, device="cuda")
    v = torch.zeros_like(k)
    ops.pa_cache_append(k, v, torch.empty((0, 2, 64), dtype=torch.float16, device="cuda"),
                        torch.empty((0, 2, 64), dtype=torch.float16, device="cuda"),
                        torch.empty((0,), dtype=torch.int32, device="cuda"))
    ops.pa_block_copy(k, v, torch.empty((0, 2), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert int(k.abs().sum()) == 0
