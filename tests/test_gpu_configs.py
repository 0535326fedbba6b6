"""End-to-end parity of the decode step on the five synthetic workloads.

Each test builds the workload on the GPU (generator + packer of the HIP
library), runs one step exactly as bench.py times it, and checks sampled rows
against the oracle, which draws the same rows with the host generator:
indexer scores, block maxima, the pool and the top-512 bit-exact; the
sparse-branch output, its log-sum-exp and the merged output within
|o - ref| <= 2e-3 + 1e-2 |ref|.
"""
import numpy as np
import pytest
import torch

from long_context_sparse_amd.workload import Workload
from synth import configs
from tests.ref import RowRef

pytestmark = pytest.mark.gpu


def tol_ok(got, ref):
    return bool(np.all(np.abs(got - ref) <= 2e-3 + 1e-2 * np.abs(ref)))


def check_attention(wl, layer_i, row, ref, idx):
    o_p, lse_p, o = ref.attend(idx)
    L = wl.layers[layer_i]
    n = int(L.idx_count[row])
    assert np.array_equal(L.idx[row, :n].cpu().numpy(), idx)
    if wl.separate:
        assert tol_ok(L.o_partial[row].cpu().numpy(), o_p)
        assert np.allclose(L.lse[row].cpu().numpy(), lse_p, rtol=1e-5, atol=1e-4)
    assert tol_ok(L.out[row].cpu().numpy(), o)


def check_full_row(wl, row):
    ref = RowRef(wl.cfg, row, 0)
    scores = ref.full_scores()
    got = wl.scores[row, :ref.n_vis].cpu().numpy()
    assert np.array_equal(got, scores), np.nonzero(got != scores)[0][:5]
    nb = (ref.n_vis + 7) // 8
    import oracle
    assert np.array_equal(wl.block_max[row, :nb].cpu().numpy(), oracle.block_max(scores))
    pool, idx = ref.select_full(scores)
    assert int(wl.pool_count[row]) == len(pool)
    assert np.array_equal(wl.pool[row, :len(pool)].cpu().numpy(), pool)
    check_attention(wl, 0, row, ref, idx)
    return pool


@pytest.fixture(scope="module")
def tiny():
    wl = Workload(configs.tiny_full_decode())
    wl.step()
    torch.cuda.synchronize()
    return wl


def test_tiny_full_decode(tiny):
    check_full_row(tiny, 0)


def test_tiny_full_decode_two_call_forms():
    """The two-call selection (blocks, then positions) and the two-call
    attention (sparse branch, then window merge) give the same results."""
    wl = Workload(configs.tiny_full_decode(), separate=True, two_call_select=True)
    wl.step()
    torch.cuda.synchronize()
    check_full_row(wl, 0)


def test_tiny_repeatable(tiny):
    before = tiny.layers[0].out.clone()
    tiny.step()
    torch.cuda.synchronize()
    assert torch.equal(before, tiny.layers[0].out)


def test_full_decode_128k_sampled_rows():
    wl = Workload(configs.full_decode_128k())
    wl.step()
    torch.cuda.synchronize()
    for row in (0, 11):
        check_full_row(wl, row)
    del wl
    torch.cuda.empty_cache()


def pool_columns(pool, n_vis, scores):
    """Scores of the pool's positions laid out by column (8 per block), -inf
    where a position of a partial last block is not visible."""
    pos = (8 * np.asarray(pool, np.int64)[:, None] + np.arange(8)).reshape(-1)
    out = np.full(len(pos), -np.inf, np.float32)
    out[pos < n_vis] = scores
    return out


def check_reindex_row(wl, layer_i, row, pool, check_scores):
    ref = RowRef(wl.cfg, row, layer_i)
    pos, sc, idx = ref.select_pool(pool)
    if check_scores:
        got = wl.pool_scores[row, :8 * len(pool)].cpu().numpy()
        assert np.array_equal(got, pool_columns(pool, ref.n_vis, sc))
    check_attention(wl, layer_i, row, ref, idx)


def test_reindex_decode_1m_sampled_rows():
    """64 requests x 1,048,576 entries, given pools, boosted keys: the pool
    re-scoring, the top-512 and the attention of three rows."""
    cfg = configs.reindex_decode_1m()
    wl = Workload(cfg)
    wl.step()
    torch.cuda.synchronize()
    import synth
    for row in (0, 31, 63):
        pool = synth.given_pool(cfg.seed, row, int(cfg.lens[row]) // 8, 2048)
        assert np.array_equal(wl.pool[row].cpu().numpy(), pool)
        check_reindex_row(wl, 0, row, pool, check_scores=True)
    del wl
    torch.cuda.empty_cache()


def test_chunked_prefill_sampled_rows():
    """4,096 causal query rows over 131,072 entries (2 tokens per entry):
    every visible score, the block maxima, the top-512 and the attention of
    the first, a middle and the last row."""
    cfg = configs.chunked_prefill_256k()
    wl = Workload(cfg)
    wl.step()
    torch.cuda.synchronize()
    import oracle
    for row in (0, 2047, 4095):
        ref = RowRef(cfg, row, 0)
        scores = ref.full_scores()
        got = wl.scores[row, :ref.n_vis].cpu().numpy()
        assert np.array_equal(got, scores), (row, np.nonzero(got != scores)[0][:5])
        nb = (ref.n_vis + 7) // 8
        assert np.array_equal(wl.block_max[row, :nb].cpu().numpy(), oracle.block_max(scores))
        check_attention(wl, 0, row, ref, ref.select_prefill(scores))
    del wl
    torch.cuda.empty_cache()


def test_mixed_serving_sampled_rows():
    """256 ragged requests in 64-entry pages in random order; one Full layer
    builds the pools, four Reindex layers re-score them.  The shortest, a
    middle and the longest (1,047,075 entries) request through all layers."""
    cfg = configs.mixed_serving()
    wl = Workload(cfg)
    wl.step()
    torch.cuda.synchronize()
    L = cfg.lens
    order = np.argsort(L, kind="stable")
    last = len(wl.layers) - 1
    for row in (int(order[0]), int(order[len(order) // 2]), int(order[-1])):
        pool = check_full_row(wl, row)
        for li in range(1, len(wl.layers)):
            check_reindex_row(wl, li, row, pool, check_scores=li == last)
    del wl
    torch.cuda.empty_cache()
