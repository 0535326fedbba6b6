"""End-to-end parity of the decode step on the five synthetic workloads.

Each test builds the workload on the GPU (generator + packer of the HIP
library), runs one step exactly as bench.py times it, and checks it against
the oracle, which draws the same rows with the host generator:

* every row of every layer: cheap invariants that any correct step meets --
  pool and index counts (min(2,048, blocks), min(512, candidates)), ids
  strictly ascending, inside the row's visible range and its pool, padding
  -1, outputs and log-sum-exps finite;
* rows checked against the oracle (all of them for the two decode
  workloads, a spread of rows for the prefill and mixed ones): indexer
  scores, block maxima, the pool and the top-512 bit-exact; the output within
  |o - ref| <= 2e-3 + 1e-2 |ref| (and the sparse branch, where the step runs
  the two-call form).
The oracle rows run on a thread pool, one row per thread.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from long_context_sparse_amd.workload import Workload
from synth import configs
from tests.ref import RowRef

pytestmark = pytest.mark.gpu


def tol_ok(got, ref):
    return bool(np.all(np.abs(got - ref) <= 2e-3 + 1e-2 * np.abs(ref)))


# ---------------------------------------------------------------- every row
def _ids_ok(ids, count, width, upper):
    """ids[:count] strictly ascending in [0, upper), the rest of `width` -1."""
    v = ids[:count]
    return (len(v) == count and np.all(v >= 0) and np.all(v < upper) and np.all(np.diff(v) > 0)
            and np.all(ids[count:width] == -1))


def check_invariants(wl, n_pool=2048):
    """Every row of every layer of the step just run."""
    nv = wl.n_vis_host
    nb = (nv + 7) // 8
    pool = wl.pool.cpu().numpy()
    pc = wl.pool_count.cpu().numpy()
    reindex_only = wl.cfg.mode == "reindex"
    if not reindex_only:
        assert np.array_equal(pc, np.minimum(nb, n_pool)), "pool counts"
    for r in range(wl.n_rows):
        assert _ids_ok(pool[r], pc[r], pool.shape[1], nb[r]), ("pool", r)
    sel_role = None
    for li, L in enumerate(wl.layers):
        idx, ic = L.idx.cpu().numpy(), L.idx_count.cpu().numpy()
        # candidates of a row: its visible pool positions (Full: every position
        # of the pool blocks; the prefill's 512-block pool holds >= 512 of
        # them); a Reuse layer shares the positions of the layer before it
        sel_role = L.role if L.role != "reuse" else sel_role
        cand = np.minimum(8 * pc, nv) if sel_role == "reindex" else nv
        assert np.array_equal(ic, np.minimum(cand, 512)), ("idx counts", li)
        for r in range(wl.n_rows):
            assert _ids_ok(idx[r], ic[r], idx.shape[1], nv[r]), ("idx", li, r)
            if wl.cfg.mode != "prefill":
                assert np.all(np.isin(idx[r, :ic[r]] // 8, pool[r, :pc[r]])), ("idx outside the pool", li, r)
        out = L.out.cpu().numpy()
        assert np.all(np.isfinite(out)), ("non-finite output", li)


# ---------------------------------------------------------------- oracle rows
def _full_ref(cfg, row, chunk=1 << 30):
    """Oracle of one row of a Full layer (scores of every position, pool,
    top-512, attention); rows longer than `chunk` score their positions in
    chunks on a thread pool."""
    ref = RowRef(cfg, row, 0)
    scores = ref.scores_at(np.arange(ref.n_vis), chunk=chunk)
    pool, idx = ref.select_full(scores)
    o_p, lse_p, o = ref.attend(idx)
    return dict(ref=ref, scores=scores, pool=pool, idx=idx, o_p=o_p, lse_p=lse_p, o=o)


def _reindex_ref(cfg, row, layer, pool):
    ref = RowRef(cfg, row, layer)
    pos = oracle.pool_positions(pool, ref.n_vis)
    sc = ref.scores_at(pos, chunk=1 << 30)
    idx = oracle.topk(sc, 512, ids=pos)
    o_p, lse_p, o = ref.attend(idx)
    return dict(ref=ref, pos=pos, scores=sc, idx=idx, o_p=o_p, lse_p=lse_p, o=o)


def compare_attention(wl, layer_i, row, d):
    L = wl.layers[layer_i]
    n = int(L.idx_count[row])
    assert np.array_equal(L.idx[row, :n].cpu().numpy(), d["idx"]), ("idx", layer_i, row)
    if wl.separate:
        assert tol_ok(L.o_partial[row].cpu().numpy(), d["o_p"]), ("sparse branch", layer_i, row)
        assert np.allclose(L.lse[row].cpu().numpy(), d["lse_p"], rtol=1e-5, atol=1e-4)
    got = L.out[row].cpu().numpy()
    assert tol_ok(got, d["o"]), ("output", layer_i, row, float(np.abs(got - d["o"]).max()))


def compare_full_row(wl, row, d):
    n_vis = d["ref"].n_vis
    got = wl.scores[row, :n_vis].cpu().numpy()
    assert np.array_equal(got, d["scores"]), ("scores", row, np.nonzero(got != d["scores"])[0][:5])
    nb = (n_vis + 7) // 8
    assert np.array_equal(wl.block_max[row, :nb].cpu().numpy(), oracle.block_max(d["scores"])), ("block max", row)
    pool = d["pool"]
    assert int(wl.pool_count[row]) == len(pool)
    assert np.array_equal(wl.pool[row, :len(pool)].cpu().numpy(), pool), ("pool", row)
    compare_attention(wl, 0, row, d)


def pool_columns(pool, n_vis, scores):
    """Scores of the pool's positions laid out by column (8 per block), -inf
    where a position of a partial last block is not visible."""
    pos = (8 * np.asarray(pool, np.int64)[:, None] + np.arange(8)).reshape(-1)
    out = np.full(len(pos), -np.inf, np.float32)
    out[pos < n_vis] = scores
    return out


def compare_reindex_row(wl, layer_i, row, pool, d, check_scores):
    if check_scores:
        got = wl.pool_scores[row, :8 * len(pool)].cpu().numpy()
        assert np.array_equal(got, pool_columns(pool, d["ref"].n_vis, d["scores"])), ("pool scores", row)
    compare_attention(wl, layer_i, row, d)


# ---------------------------------------------------------------- workloads
@pytest.fixture(scope="module")
def tiny():
    wl = Workload(configs.tiny_full_decode())
    wl.step()
    torch.cuda.synchronize()
    return wl


def test_tiny_full_decode(tiny):
    check_invariants(tiny)
    compare_full_row(tiny, 0, _full_ref(tiny.cfg, 0))


def test_tiny_full_decode_two_call_forms():
    """The two-call selection (blocks, then positions) and the two-call
    attention (sparse branch, then window merge) give the same results."""
    wl = Workload(configs.tiny_full_decode(), separate=True, two_call_select=True)
    wl.step()
    torch.cuda.synchronize()
    check_invariants(wl)
    compare_full_row(wl, 0, _full_ref(wl.cfg, 0))


def test_tiny_repeatable(tiny):
    before = tiny.layers[0].out.clone()
    tiny.step()
    torch.cuda.synchronize()
    assert torch.equal(before, tiny.layers[0].out)


def test_full_decode_128k_every_row():
    """16 requests x 131,072 entries: every row against the oracle."""
    cfg = configs.full_decode_128k()
    wl = Workload(cfg)
    wl.step()
    torch.cuda.synchronize()
    check_invariants(wl)
    refs = oracle.map_rows(lambda r: _full_ref(cfg, r), list(range(wl.n_rows)))
    for row, d in enumerate(refs):
        compare_full_row(wl, row, d)
    del wl
    torch.cuda.empty_cache()


def test_reindex_decode_1m_every_row():
    """64 requests x 1,048,576 entries, given pools, boosted keys: every
    row's pool re-scoring, top-512 and attention against the oracle."""
    cfg = configs.reindex_decode_1m()
    wl = Workload(cfg)
    wl.step()
    torch.cuda.synchronize()
    check_invariants(wl)
    pools = [synth.given_pool(cfg.seed, r, int(cfg.lens[r]) // 8, 2048) for r in range(wl.n_rows)]
    got_pools = wl.pool.cpu().numpy()
    for r in range(wl.n_rows):
        assert np.array_equal(got_pools[r], pools[r])
    refs = oracle.map_rows(lambda r: _reindex_ref(cfg, r, 0, pools[r]), list(range(wl.n_rows)))
    for row, d in enumerate(refs):
        compare_reindex_row(wl, 0, row, pools[row], d, check_scores=True)
    del wl
    torch.cuda.empty_cache()


def test_chunked_prefill_rows():
    """4,096 causal query rows over 131,072 entries (2 tokens per entry):
    invariants on every row; every visible score, the block maxima, the
    top-512 and the attention of eight rows (first, last, a spread between)."""
    cfg = configs.chunked_prefill_256k()
    wl = Workload(cfg)
    wl.step()
    torch.cuda.synchronize()
    check_invariants(wl, n_pool=512)
    rows = [0, 1, 517, 1366, 2047, 3001, 4094, 4095]

    def job(row):
        ref = RowRef(cfg, row, 0)
        scores = ref.scores_at(np.arange(ref.n_vis), chunk=1 << 30)
        idx = ref.select_prefill(scores)
        o_p, lse_p, o = ref.attend(idx)
        return dict(ref=ref, scores=scores, idx=idx, o_p=o_p, lse_p=lse_p, o=o)

    for row, d in zip(rows, oracle.map_rows(job, rows)):
        n_vis = d["ref"].n_vis
        got = wl.scores[row, :n_vis].cpu().numpy()
        assert np.array_equal(got, d["scores"]), (row, np.nonzero(got != d["scores"])[0][:5])
        nb = (n_vis + 7) // 8
        assert np.array_equal(wl.block_max[row, :nb].cpu().numpy(), oracle.block_max(d["scores"]))
        compare_attention(wl, 0, row, d)
    del wl
    torch.cuda.empty_cache()


def test_mixed_serving_rows():
    """256 ragged requests in 64-entry pages in random order; one Full layer
    builds the pools, four Reindex layers re-score them.  Invariants on every
    request and layer; six requests (the shortest, the longest at 1,047,075
    entries, the median and three more) through all layers against the
    oracle."""
    cfg = configs.mixed_serving()
    wl = Workload(cfg)
    wl.step()
    torch.cuda.synchronize()
    check_invariants(wl)
    order = np.argsort(cfg.lens, kind="stable")
    rows = sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1]), 7, 100, 201})
    full = {r: _full_ref(cfg, r, chunk=1 << 15) for r in rows}      # long rows: chunks in parallel
    for row in rows:
        compare_full_row(wl, row, full[row])
    last = len(wl.layers) - 1
    jobs = [(li, row) for li in range(1, len(wl.layers)) for row in rows]
    reidx = oracle.map_rows(lambda j: _reindex_ref(cfg, j[1], j[0], full[j[1]]["pool"]), jobs)
    for (li, row), d in zip(jobs, reidx):
        compare_reindex_row(wl, li, row, full[row]["pool"], d, check_scores=li == last)
    del wl
    torch.cuda.empty_cache()


def test_decoder_stack_rows():
    """The decoder's 20 layers at 16 x 131,072 entries: one Full layer, four
    Reindex layers, each followed by three Reuse layers that attend with their
    own query and window over the positions just selected ('KV cache diet'
    page, figure 2; V4.1 Flash architecture page: a Reuse layer still runs
    attention with its own query).  Invariants on every row and layer; three
    rows through all 20 layers against the oracle."""
    cfg = configs.decoder_stack_128k()
    wl = Workload(cfg)
    wl.step()
    torch.cuda.synchronize()
    check_invariants(wl)
    rows = [0, 7, 15]
    full = dict(zip(rows, oracle.map_rows(lambda r: _full_ref(cfg, r), rows)))
    for row in rows:
        compare_full_row(wl, row, full[row])
    jobs, src = [], {row: full[row]["idx"] for row in rows}
    for li, L in enumerate(wl.layers):
        if li == 0:
            continue
        for row in rows:
            jobs.append((li, L.role, row))
    # the Reindex layers first (their selections feed the Reuse layers after them)
    reidx = {(li, row): _reindex_ref(cfg, row, li, full[row]["pool"]) for li, role, row in jobs if role == "reindex"}
    sources = {}
    for li, L in enumerate(wl.layers):
        for row in rows:
            if L.role == "reindex":
                src[row] = reidx[(li, row)]["idx"]
            sources[(li, row)] = src[row]

    def reuse(j):
        li, _, row = j
        _, _, o = RowRef(cfg, row, li).attend(sources[(li, row)])
        return o

    reuse_jobs = [j for j in jobs if j[1] == "reuse"]
    reuse_out = dict(zip(reuse_jobs, oracle.map_rows(reuse, reuse_jobs)))
    for li, role, row in jobs:
        L = wl.layers[li]
        if role == "reindex":
            compare_reindex_row(wl, li, row, full[row]["pool"], reidx[(li, row)], check_scores=li == 16)
        else:
            n = int(L.idx_count[row])
            assert np.array_equal(L.idx[row, :n].cpu().numpy(), sources[(li, row)])
            got = L.out[row].cpu().numpy()
            o = reuse_out[(li, role, row)]
            assert tol_ok(got, o), ("reuse output", li, row, float(np.abs(got - o).max()))
    del wl
    torch.cuda.empty_cache()


def test_graph_replay_matches_eager():
    """A whole step captured as a HIP graph (per KV copy) and replayed:
    every replay, with eager work and a synchronisation between replays,
    gives the eager step's bits for every layer's scores, pool, positions and
    outputs (8 layers: Full, Reindex and Reuse; 4 requests x 20,000 entries,
    two KV copies)."""
    from synth.configs import Config
    roles = ("full", "reuse", "reuse", "reuse", "reindex", "reuse", "reuse", "reuse")
    cfg = Config("graph_check", seed=9, n_req=4, heads=64, ctx=20000, mode="full", layer_roles=roles)
    wl = Workload(cfg, copies=2)

    def snapshot():
        t = [wl.scores, wl.block_max, wl.pool, wl.pool_count, wl.pool_scores]
        for L in wl.layers:
            t += [L.idx, L.idx_count, L.out]
        return [x.clone() for x in t]

    wl.step(copy=1)
    torch.cuda.synchronize()
    ref = snapshot()
    wl.capture_graphs()
    for rep in range(3):
        for x in [wl.scores, wl.block_max, wl.pool_scores] + [L.out for L in wl.layers]:
            x.fill_(float("nan"))
        for x in [wl.pool, wl.pool_count] + [L.idx for L in wl.layers]:
            x.fill_(-5)
        torch.cuda.synchronize()
        wl.replay(copy=1)
        torch.cuda.synchronize()
        got = snapshot()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), (rep, i)
        wl.replay(copy=0)            # the other copy holds the same cache: same bits
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(snapshot(), ref)):
            assert torch.equal(a, b), (rep, "copy 0", i)
    _, _, o = RowRef(cfg, 2, 7).attend(RowRef(cfg, 2, 4).select_pool(
        wl.pool[2, :int(wl.pool_count[2])].cpu().numpy())[2])
    assert tol_ok(wl.layers[7].out[2].cpu().numpy(), o)


def test_hca_decode_rows():
    """The heavily compressed branch ('DeepSeek-V4' page, section 2.3.2): 16
    requests of 1,048,576 tokens at 128 tokens per entry, every one of the
    8,192 entries attended densely with the window and a per-head sink
    (section 2.3.3).  Every row finite; three rows against the oracle."""
    cfg = configs.hca_decode_1m()
    wl = Workload(cfg)
    wl.step()
    torch.cuda.synchronize()
    L = wl.layers[0]
    out = L.out.cpu().numpy()
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(L.lse.cpu().numpy()))
    rows = [0, 6, 15]
    refs = oracle.map_rows(lambda r: RowRef(cfg, r, 0).attend_dense(), rows)
    for row, o in zip(rows, refs):
        assert tol_ok(out[row], o), (row, float(np.abs(out[row] - o).max()))
    del wl
    torch.cuda.empty_cache()


def test_v4_csa_decode_rows():
    """The compressed sparse attention of the V4 hybrid ('DeepSeek-V4' page,
    sections 2.3.1 and 4.2.1): 16 requests of 1,048,576 tokens at 4 tokens
    per entry (262,144 entries), 64 indexer heads, the top-512 over every
    visible entry, the window and a per-head sink.  Invariants on every row;
    three rows' scores, block maxima, top-512 and output against the oracle."""
    cfg = configs.v4_csa_decode_1m()
    wl = Workload(cfg)
    wl.step()
    torch.cuda.synchronize()
    check_invariants(wl, n_pool=512)
    rows = [0, 9, 15]

    def job(row):
        ref = RowRef(cfg, row, 0)
        scores = ref.scores_at(np.arange(ref.n_vis), chunk=1 << 15)
        idx = ref.select_prefill(scores)      # the top-512 of every visible score
        o_p, lse_p, o = ref.attend(idx, sink=ref.sink)
        return dict(ref=ref, scores=scores, idx=idx, o_p=o_p, lse_p=lse_p, o=o)

    for row in rows:
        d = job(row)
        n_vis = d["ref"].n_vis
        got = wl.scores[row, :n_vis].cpu().numpy()
        assert np.array_equal(got, d["scores"]), (row, np.nonzero(got != d["scores"])[0][:5])
        nb = (n_vis + 7) // 8
        assert np.array_equal(wl.block_max[row, :nb].cpu().numpy(), oracle.block_max(d["scores"]))
        compare_attention(wl, 0, row, d)
    del wl
    torch.cuda.empty_cache()
