"""Pins the oracle's top-k, block maximum and the Full / Reindex selection.

Definitions: top-k selector of the 'DeepSeek-V4' paper page, section 2.3.1
(C_t = {C_s : I_{t,s} in Top-k(I_{t,:})}, k = 512 'index_topk'); hierarchical
sparse indexer of the V4.1-Flash architecture page (positions grouped by 8,
a group ranked by its maximum score, up to 2,048 groups kept; Reindex layers
pick their own top-512 inside the 16,384-position pool); ties go to the lower
position.

Pins: brute force with Python's sorted() on keys with many duplicates;
k >= n; the block maximum against a numpy reshape; the invariant that the
Full layer's top-512 inside the pool equals the global top-512; pool size
min(2048, ceil(n/8)); Reindex over the full block set equals Full.
"""
import numpy as np
import pytest

RNG = np.random.default_rng(31)


def brute_topk(keys, k, ids=None):
    ids = list(range(len(keys))) if ids is None else [int(i) for i in ids]
    order = sorted(zip(keys.tolist(), ids), key=lambda t: (-t[0], t[1]))
    return np.array(sorted(i for _, i in order[:k]), np.int32)


@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (100, 100), (100, 150), (1000, 17), (5000, 512), (16384, 2048)])
def test_topk_brute_force(orc, n, k):
    keys = RNG.integers(0, 40, n).astype(np.float32) * 0.25     # heavy ties
    assert np.array_equal(orc.topk(keys, k), brute_topk(keys, k))
    ids = RNG.permutation(10 * n)[:n].astype(np.int32)
    assert np.array_equal(orc.topk(keys, k, ids), brute_topk(keys, k, ids))


def test_topk_empty_and_signed(orc):
    assert len(orc.topk(np.zeros(0, np.float32), 5)) == 0
    keys = np.array([-1.0, 0.0, -0.5, 3.0, -7.0], np.float32)
    assert np.array_equal(orc.topk(keys, 3), np.array([1, 2, 3]))


@pytest.mark.parametrize("n", [1, 8, 13, 4096, 20000])
def test_block_max(orc, n):
    s = RNG.standard_normal(n).astype(np.float32)
    pad = np.full(((n + 7) // 8) * 8, -np.inf, np.float32)
    pad[:n] = s
    assert np.array_equal(orc.block_max(s), pad.reshape(-1, 8).max(1))


@pytest.mark.parametrize("n", [4096, 20000, 131072])
def test_full_select_invariants(orc, n):
    scores = np.abs(RNG.standard_normal(n)).astype(np.float32)
    scores[RNG.integers(0, n, n // 10)] = 1.0     # ties
    pool, idx = orc.full_select(scores)
    assert len(pool) == min(2048, (n + 7) // 8)
    assert np.all(np.diff(pool) > 0) and np.all(np.diff(idx) > 0)
    # the top-512 inside the pool is the global top-512
    assert np.array_equal(idx, brute_topk(scores, 512))
    assert set((idx // 8).tolist()) <= set(pool.tolist())
    # the pool is the brute-force top-2048 of the block maxima
    bm = np.array([scores[8 * j:8 * j + 8].max() for j in range((n + 7) // 8)], np.float32)
    assert np.array_equal(pool, brute_topk(bm, 2048))


def test_reindex_all_blocks_equals_full(orc):
    n = 4096
    scores = RNG.standard_normal(n).astype(np.float32)
    all_blocks = np.arange(n // 8, dtype=np.int32)
    pos = orc.pool_positions(all_blocks, n)
    assert np.array_equal(pos, np.arange(n))
    assert np.array_equal(orc.topk(scores[pos], 512, pos), orc.full_select(scores)[1])
