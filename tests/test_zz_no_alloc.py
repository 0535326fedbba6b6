"""The allocation-free attention entry point (csa2_sparse_swa_attn_noalloc)
against the workspace form of csa2_sparse_swa_attn, through the C ABI: the
same bits (outputs and log-sum-exps) on two calls in a row, the second with a
smaller input, so the library's scratch carries the first call's partials
into the second."""
import numpy as np
import pytest
import torch

import long_context_sparse_amd as lib
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"
SIG = 512 ** -0.5


def _case(rng, n_rows, H, n_entries):
    lat = torch.as_tensor(rng.standard_normal((n_rows * n_entries, 512)).astype(np.float32)).bfloat16().float()
    mc, ms = oracle.pack_main(lat.numpy())
    swa = torch.as_tensor(rng.standard_normal((n_rows * 128, 512)).astype(np.float32)).bfloat16().float()
    wc, wsc = oracle.pack_swa(swa.numpy())
    q = torch.as_tensor(rng.standard_normal((n_rows, H, 512)).astype(np.float32)).bfloat16().to(DEV)
    counts = rng.integers(1, 513, n_rows).astype(np.int32)
    counts[0] = 512
    swa_counts = rng.integers(0, 129, n_rows).astype(np.int32)
    swa_counts[0] = 128
    idx = np.full((n_rows, 512), -1, np.int32)
    for r in range(n_rows):
        idx[r, :counts[r]] = np.sort(rng.permutation(n_entries)[:counts[r]])
    T = lambda a: torch.as_tensor(np.ascontiguousarray(a)).to(DEV)   # noqa: E731
    kv = lib.make_kv(main_codes=T(mc), main_scales=T(ms), n_slots=n_rows * n_entries, req_stride=n_entries)
    rows = lib.make_rows(T(np.arange(n_rows, dtype=np.int32)), T(np.full(n_rows, n_entries, np.int32)), n_entries)
    sink = T((rng.standard_normal(H) * 2).astype(np.float32))
    args = (kv, rows, q, T(idx), T(counts), T(wc), T(wsc), T(np.arange(n_rows, dtype=np.int64) * 128),
            T(swa_counts), SIG)
    return args, sink


def _both(args, sink, n_rows, H):
    wsb = lib.csa2_attn_workspace_size(n_rows, H)
    assert wsb > 0, "the shape must take the split pass"
    ws = torch.empty(wsb // 4, dtype=torch.float32, device=DEV)
    out_ref = torch.empty((n_rows, H, 512), dtype=torch.float32, device=DEV)
    lse_ref = torch.empty((n_rows, H), dtype=torch.float32, device=DEV)
    lib.csa2_sparse_swa_attn(*args, out_ref, sink=sink, lse=lse_ref, workspace=ws)
    out = torch.full((n_rows, H, 512), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((n_rows, H), float("nan"), dtype=torch.float32, device=DEV)
    lib.csa2_sparse_swa_attn_noalloc(*args, out, sink=sink, lse=lse)
    torch.cuda.synchronize()
    return out, lse, out_ref, lse_ref


def test_noalloc_matches_workspace_form():
    rng = np.random.default_rng(77)
    # first call: 16 rows x 64 heads (4 splits per row and head group)
    args, sink = _case(rng, 16, 64, 600)
    out, lse, out_ref, lse_ref = _both(args, sink, 16, 64)
    assert torch.equal(out, out_ref) and torch.equal(lse, lse_ref)
    # second call, smaller: 3 rows x 16 heads
    args, sink = _case(rng, 3, 16, 520)
    out, lse, out_ref, lse_ref = _both(args, sink, 3, 16)
    assert torch.equal(out, out_ref) and torch.equal(lse, lse_ref)
    assert bool(torch.isfinite(out).all())
