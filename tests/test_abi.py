"""The C-ABI boundary without a GPU: the library loads, exports every entry
point include/csa2.h declares, and rejects bad arguments on the host before
any launch (status code + message, nothing enqueued)."""
import ctypes
import os
import re

import pytest

import long_context_sparse_amd as lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "csa2.h")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = lib.lib()
    names = declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(lib.EXPORTS)
    assert L.csa2_abi_version() == 5


def _kv(**over):
    kv = lib.KV(256, 256, 256, 256, 1000, 0, 0, None, 1000)
    for k, v in over.items():
        setattr(kv, k, v)
    return kv


def _rows(n=2, max_vis=100):
    return lib.Rows(256, 512, n, max_vis)


def test_status_strings():
    L = lib.lib()
    for s in range(8):
        assert L.csa2_status_str(s)


def _topk(L, keys=256, key_stride=100, ids=None, ids_stride=0, n_cols=None, mul=1, div=1, pool=None,
          pool_stride=0, by_id=0, n_rows=4, max_cols=100, k=10, out=256, out_stride=16, cnt=256, ws=None,
          ws_bytes=0):
    return L.csa2_select_topk(keys, key_stride, ids, ids_stride, n_cols, mul, div, pool, pool_stride, by_id,
                              n_rows, max_cols, k, out, out_stride, cnt, ws, ws_bytes, None)


@pytest.mark.parametrize("k,expect", [(0, 3), (2049, 3)])
def test_topk_rejects_k(k, expect):
    L = lib.lib()
    assert _topk(L, k=k, out_stride=2048) == expect
    assert b"k must be" in L.csa2_last_error()


def test_topk_rejects_shapes():
    """Every call here is invalid (nothing is launched), except the one with
    no rows."""
    L = lib.lib()
    assert _topk(L, keys=None) == 1
    assert _topk(L, out_stride=5) == 2                              # out_stride < k
    assert _topk(L, by_id=1) == 2                                   # keys_by_id without a pool
    assert _topk(L, key_stride=50) == 2                             # key_stride < max_cols
    assert _topk(L, mul=9) == 3
    assert _topk(L, ids=512, ids_stride=100, pool=768, pool_stride=16) == 2   # ids and pool exclusive
    assert _topk(L, ids=512, ids_stride=99) == 2                    # ids_stride < max_cols
    assert _topk(L, ws=None, ws_bytes=64) == 1                      # size without a workspace
    assert _topk(L, ws=264, ws_bytes=64) == 4                       # workspace alignment
    # zero rows: nothing to do
    assert _topk(L, keys=None, key_stride=0, n_rows=0, max_cols=0, out=None, out_stride=0, cnt=None) == 0


def test_topk_workspace_size():
    L = lib.lib()
    for n_rows, max_cols, k in ((1, 1, 1), (64, 16384, 512), (4096, 131072, 2048)):
        assert L.csa2_select_topk_workspace(n_rows, max_cols, k) == 0


def test_select_full_rejects():
    L = lib.lib()
    f = L.csa2_select_full
    ok = (256, 16, 256, 128, 256, 4, 100, 2048, 512, 256, 2048, 256, 256, 512, 256, None)   # never launched
    bad = list(ok); bad[7] = 2049                   # pool too large
    assert f(*bad) == 3
    bad = list(ok); bad[8] = 0                      # k
    assert f(*bad) == 3
    bad = list(ok); bad[0] = None                   # block_max
    assert f(*bad) == 1
    bad = list(ok); bad[3] = 100                    # scores_stride < roundup(max_vis, 8)
    assert f(*bad) == 2
    bad = list(ok); bad[1] = 12                     # block_max_stride < ceil(max_vis / 8)
    assert f(*bad) == 2
    bad = list(ok); bad[2] = 260                    # scores not 16-byte aligned
    assert f(*bad) == 4
    bad = list(ok); bad[13] = 100                   # idx_stride < k
    assert f(*bad) == 2
    assert f(None, 0, None, 0, None, 0, 0, 2048, 512, None, 0, None, None, 0, None, None) == 0   # no rows


def test_pack_rejects():
    L = lib.lib()
    assert L.csa2_pack_kv(7, 256, 0, 4, 512, 256, 256, None, None) == 5
    assert L.csa2_pack_kv(0, 256, 5, 4, 512, 256, 256, None, None) == 5
    assert L.csa2_pack_kv(0, None, 0, 4, 512, 256, 256, None, None) == 1
    assert L.csa2_pack_kv(0, 256, 0, 4, 100, 256, 256, None, None) == 2
    assert L.csa2_pack_kv(0, 258, 0, 4, 512, 256, 256, None, None) == 4
    assert L.csa2_pack_kv(0, 256, 0, 4, 512, 272, 256, None, None) == 4
    assert L.csa2_pack_kv(0, 256, 0, -1, 512, 256, 256, None, None) == 3
    assert L.csa2_pack_kv(0, None, 0, 0, 512, None, None, None, None) == 0


def test_index_score_rejects():
    L = lib.lib()
    kv, rows = _kv(), _rows()
    f = L.csa2_index_score
    B = ctypes.byref
    assert f(None, B(rows), 256, 0, 8, 256, None, 0, None, 256, 104, None, 0, None) == 1
    assert f(B(kv), B(rows), 256, 0, 65, 256, None, 0, None, 256, 104, None, 0, None) == 5    # 65 heads
    assert f(B(kv), B(rows), 256, 0, 0, 256, None, 0, None, 256, 104, None, 0, None) == 5
    assert f(B(kv), B(rows), 256, 0, 8, 256, None, 0, None, 256, 99, None, 0, None) == 2
    assert f(B(kv), B(rows), 256, 0, 8, 256, None, 0, None, None, 0, None, 0, None) == 1
    assert f(B(_kv(idx_codes=300)), B(rows), 256, 0, 8, 256, None, 0, None, 256, 104, None, 0, None) == 4
    assert f(B(_kv(page_entries=48, page_table=256, max_pages=4)), B(rows), 256, 0, 8, 256, None, 0, None,
             256, 104, None, 0, None) == 3
    assert f(B(_kv(page_entries=64)), B(rows), 256, 0, 8, 256, None, 0, None, 256, 104, None, 0, None) == 1
    # pool mode needs pool_count and forbids block_max
    assert f(B(kv), B(rows), 256, 0, 8, 256, 256, 2048, None, 256, 16384, None, 0, None) == 1
    assert f(B(kv), B(rows), 256, 0, 8, 256, 256, 2048, 256, 256, 16384, 256, 2048, None) == 2


def test_index_score_shared_rejects():
    """Argument errors of the shared-request scan return before any launch
    (every call here is invalid, so nothing is enqueued)."""
    L = lib.lib()
    kv, rows = _kv(), _rows()
    f = L.csa2_index_score_shared
    B = ctypes.byref
    assert f(None, B(rows), 0, 256, 0, 8, 256, 256, 104, None, 0, None) == 1            # no cache
    assert f(B(kv), None, 0, 256, 0, 8, 256, 256, 104, None, 0, None) == 1              # no rows
    assert f(B(kv), B(rows), -1, 256, 0, 8, 256, 256, 104, None, 0, None) == 3          # req < 0
    assert f(B(kv), B(rows), 0, 256, 0, 17, 256, 256, 104, None, 0, None) == 5          # 17 heads
    assert f(B(kv), B(rows), 0, 256, 0, 8, 256, 256, 99, None, 0, None) == 2            # stride
    assert f(B(kv), B(rows), 0, 256, 0, 8, 256, None, 0, None, 0, None) == 1            # no output
    assert f(B(kv), B(rows), 0, 300, 0, 8, 256, 256, 104, None, 0, None) == 4           # q alignment
    assert f(B(kv), B(rows), 0, None, 0, 8, 256, 256, 104, None, 0, None) == 1          # no query
    assert f(B(kv), B(_rows(n=70000)), 0, 256, 0, 8, 256, 256, 104, None, 0, None) == 3
    assert L.csa2_last_error()


def test_attn_rejects():
    L = lib.lib()
    kv, rows = _kv(), _rows()
    B = ctypes.byref
    f = L.csa2_sparse_attn
    F = ctypes.c_float(0.04)
    assert f(B(kv), B(rows), 256, 0, 40, 256, 512, 256, F, 256, 256, None, 0, None) == 5          # heads
    assert f(B(kv), B(rows), 256, 0, 64, 256, 512, 256, ctypes.c_float(-1.0), 256, 256, None, 0, None) == 3
    assert f(B(kv), B(rows), 256, 0, 64, 256, 512, 256, F, None, 256, None, 0, None) == 1          # o_partial
    assert f(B(kv), B(rows), 256, 0, 64, 256, 512, 256, F, 260, 256, None, 0, None) == 4           # alignment
    assert f(B(kv), B(rows), 256, 0, 64, 256, 512, 256, F, 256, 256, 300, 4096, None) == 4         # workspace
    assert f(B(_kv(main_codes=None)), B(rows), 256, 0, 64, 256, 512, 256, F, 256, 256, None, 0, None) == 1
    assert L.csa2_attn_workspace_size(2, 64) > 0 and L.csa2_attn_workspace_size(4096, 64) == 0
    g = L.csa2_swa_merge
    assert g(256, 256, 10, 256, 256, 2, 256, 0, 64, F, None, 256, None, 256, None, 0, None) == 1   # o_partial, no lse
    assert g(256, 256, 10, 256, 256, 2, 256, 0, 200, F, None, None, None, 256, None, 0, None) == 5
    assert g(264, 256, 10, 256, 256, 2, 256, 0, 64, F, None, None, None, 256, None, 0, None) == 4
    assert g(256, 256, 10, 256, 256, 2, 256, 0, 64, F, None, None, None, None, None, 0, None) == 1  # out
    h = L.csa2_sparse_swa_attn
    assert h(B(kv), B(rows), 256, 0, 64, 256, 512, 256, None, 256, 10, 256, 256, None, F, 256, None, None, 0,
             None) == 1
    assert h(B(kv), B(rows), 256, 0, 64, 256, 512, 256, 256, 256, 10, 256, 256, None, F, 260, None, None, 0,
             None) == 4
    assert h(B(kv), B(rows), 256, 0, 24, 256, 512, 256, 256, 256, 10, 256, 256, None, F, 256, None, None, 0,
             None) == 5


def test_dense_attn_rejects():
    """Host checks of the dense (heavily compressed) attention; every call
    here is invalid, so nothing is launched."""
    L = lib.lib()
    kv = _kv()
    B = ctypes.byref
    F = ctypes.c_float(0.04)
    f = L.csa2_dense_swa_attn
    ok = dict(kv=B(kv), rows=B(_rows()), q=256, qd=0, H=64, swc=None, sws=None, slots=0, first=None, cnt=None,
              sink=None, scale=F, out=256, lse=None, ws=None, wsb=0)

    def call(**over):
        a = dict(ok, **over)
        return f(a["kv"], a["rows"], a["q"], a["qd"], a["H"], a["swc"], a["sws"], a["slots"], a["first"],
                 a["cnt"], a["sink"], a["scale"], a["out"], a["lse"], a["ws"], a["wsb"], None)

    assert call(H=40) == 5                                   # heads
    assert call(out=None) == 1
    assert call(out=260) == 4
    assert call(rows=B(_rows(max_vis=(1 << 22) + 1))) == 3   # above CSA2_MAX_DENSE
    assert call(swc=256, sws=256, slots=10, first=256, cnt=None) == 1   # window without counts
    assert call(kv=B(_kv(main_codes=None))) == 1
    assert L.csa2_dense_attn_workspace_size(2, 64, 8192) > 0
    assert L.csa2_dense_attn_workspace_size(2, 64, (1 << 22) + 1) == 0
    assert L.csa2_dense_attn_workspace_size(4096, 64, 8192) == 0   # enough rows: no split pass


def test_compress_pack_rejects():
    """Host checks of the write path (every call here is invalid: nothing is
    launched), and an empty call (no complete block) that does nothing."""
    L = lib.lib()
    f = L.csa2_compress_pack
    B = ctypes.byref

    def st(**over):
        d = dict(ca=256, za=256, cb=None, zb=None, ba=256, bb=None, n_tok=8, row_stride=512, m=4)
        d.update(over)
        return lib.CompressStreams(d["ca"], d["za"], d["cb"], d["zb"], d["ba"], d["bb"], d["n_tok"],
                                   d["row_stride"], d["m"])

    F = ctypes.c_float(1e-6)
    assert f(2, B(st()), None, F, 1, 0, None, 256, 256, None, None) == 5          # SWA: not compressed
    assert f(0, None, None, F, 1, 0, None, 256, 256, None, None) == 1
    assert f(0, B(st(m=0)), None, F, 1, 0, None, 256, 256, None, None) == 3
    assert f(0, B(st(m=2000)), None, F, 1, 0, None, 256, 256, None, None) == 3
    assert f(0, B(st(ca=None)), None, F, 1, 0, None, 256, 256, None, None) == 1
    assert f(0, B(st(cb=256)), None, F, 1, 0, None, 256, 256, None, None) == 1     # cb without zb, bb
    assert f(0, B(st(row_stride=500)), None, F, 1, 0, None, 256, 256, None, None) == 2
    assert f(1, B(st(row_stride=130)), None, F, 1, 0, None, 256, 256, None, None) == 2
    assert f(0, B(st(za=264)), None, F, 1, 0, None, 256, 256, None, None) == 4
    assert f(0, B(st()), None, F, 1, 0, None, 272, 256, None, None) == 4            # codes alignment
    assert f(0, B(st()), None, ctypes.c_float(-1.0), 1, 0, None, 256, 256, None, None) == 3
    assert f(0, B(st()), None, F, 1, -5, None, 256, 256, None, None) == 3
    assert f(0, B(st(n_tok=3, ca=None)), None, F, 1, 0, None, None, None, None, None) == 0   # no complete block


def test_stream_xor_rejects():
    """Host checks of the streaming-read reference (no launch on failure; a
    zero-byte call does nothing and succeeds)."""
    f = lib.lib().csa2_stream_xor
    assert f(256, 0, 256, None) == 0                 # nothing to read
    assert f(256, -16, 256, None) == 3               # range
    assert f(256, 24, 256, None) == 2                # not a multiple of 16
    assert f(None, 32, 256, None) == 1               # buf
    assert f(256, 32, None, None) == 1               # out
    assert f(264, 32, 256, None) == 4                # buf alignment
    assert f(256, 32, 258, None) == 4                # out alignment


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: asked for more it exits with status 2 and
    says why, before touching any device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and not r.stdout
