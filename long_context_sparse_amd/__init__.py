"""Python binding of libcsa2 -- the CSA2 decode hot path on MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels of
``libcsa2.so`` (see ``include/csa2.h`` for the contract of each call).
PyTorch tensors serve as owners of device memory and as the source of the
current HIP stream.  There is no fallback: if the library is missing or a
call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcsa2.so")

BF16, F32 = 0, 1
MAIN_FP4, INDEX_MXFP4, SWA_FP8 = 0, 1, 2
LATENT, INDEX_DIM, POOL_BLOCKS, BLOCK, TOPK, WINDOW = 512, 128, 2048, 8, 512, 128

# bytes per entry of each plane: (codes, scales)
PLANE_BYTES = {MAIN_FP4: (256, 32), INDEX_MXFP4: (64, 4), SWA_FP8: (512, 32)}


class Csa2Error(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


class KV(ctypes.Structure):
    _fields_ = [
        ("main_codes", ctypes.c_void_p), ("main_scales", ctypes.c_void_p),
        ("idx_codes", ctypes.c_void_p), ("idx_scales", ctypes.c_void_p),
        ("n_slots", ctypes.c_int64), ("page_entries", ctypes.c_int32),
        ("max_pages", ctypes.c_int32), ("page_table", ctypes.c_void_p),
        ("req_stride", ctypes.c_int64),
    ]


class CompressStreams(ctypes.Structure):
    _fields_ = [("ca", ctypes.c_void_p), ("za", ctypes.c_void_p), ("cb", ctypes.c_void_p), ("zb", ctypes.c_void_p),
                ("ba", ctypes.c_void_p), ("bb", ctypes.c_void_p), ("n_tok", ctypes.c_int64),
                ("row_stride", ctypes.c_int64), ("m", ctypes.c_int32)]


class Rows(ctypes.Structure):
    _fields_ = [("req", ctypes.c_void_p), ("n_vis", ctypes.c_void_p),
                ("n_rows", ctypes.c_int32), ("max_vis", ctypes.c_int32)]


_lib = None
EXPORTS = (
    "csa2_abi_version", "csa2_status_str", "csa2_last_error", "csa2_pack_kv", "csa2_compress_pack",
    "csa2_index_score",
    "csa2_index_score_shared",
    "csa2_select_topk_workspace", "csa2_select_topk", "csa2_select_full", "csa2_attn_workspace_size", "csa2_sparse_attn", "csa2_swa_merge",
    "csa2_sparse_swa_attn", "csa2_sparse_swa_attn_noalloc", "csa2_dense_attn_workspace_size",
    "csa2_dense_swa_attn", "csa2_synth_normal", "csa2_synth_uniform", "csa2_synth_boost", "csa2_stream_xor",
)


def lib():
    """Load libcsa2.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libcsa2.so not built at {LIB_PATH}: run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    L.csa2_abi_version.restype = ctypes.c_int
    L.csa2_status_str.restype = ctypes.c_char_p
    L.csa2_status_str.argtypes = [ctypes.c_int]
    L.csa2_last_error.restype = ctypes.c_char_p
    L.csa2_pack_kv.argtypes = [ctypes.c_int, P, ctypes.c_int, i64, i64, P, P, P, P]
    L.csa2_compress_pack.argtypes = [ctypes.c_int, ctypes.POINTER(CompressStreams), P, f32, i32, i64, P, P, P, P, P]
    L.csa2_index_score.argtypes = [ctypes.POINTER(KV), ctypes.POINTER(Rows), P, ctypes.c_int, i32, P,
                                   P, i64, P, P, i64, P, i64, P]
    L.csa2_index_score_shared.argtypes = [ctypes.POINTER(KV), ctypes.POINTER(Rows), i32, P, ctypes.c_int, i32, P,
                                          P, i64, P, i64, P]
    L.csa2_select_topk_workspace.restype = ctypes.c_size_t
    L.csa2_select_topk_workspace.argtypes = [i32, i32, i32]
    L.csa2_select_topk.argtypes = [P, i64, P, i64, P, i32, i32, P, i64, i32, i32, i32, i32, P, i64, P, P,
                                   ctypes.c_size_t, P]
    L.csa2_select_full.argtypes = [P, i64, P, i64, P, i32, i32, i32, i32, P, i64, P, P, i64, P, P]
    L.csa2_attn_workspace_size.restype = ctypes.c_size_t
    L.csa2_attn_workspace_size.argtypes = [i32, i32]
    L.csa2_sparse_attn.argtypes = [ctypes.POINTER(KV), ctypes.POINTER(Rows), P, ctypes.c_int, i32, P, i64, P,
                                   f32, P, P, P, ctypes.c_size_t, P]
    L.csa2_swa_merge.argtypes = [P, P, i64, P, P, i32, P, ctypes.c_int, i32, f32, P, P, P, P, P, ctypes.c_size_t, P]
    L.csa2_sparse_swa_attn.argtypes = [ctypes.POINTER(KV), ctypes.POINTER(Rows), P, ctypes.c_int, i32, P, i64, P,
                                       P, P, i64, P, P, P, f32, P, P, P, ctypes.c_size_t, P]
    L.csa2_sparse_swa_attn_noalloc.argtypes = [ctypes.POINTER(KV), ctypes.POINTER(Rows), P, ctypes.c_int, i32, P,
                                               i64, P, P, P, i64, P, P, P, f32, P, P, P]
    L.csa2_dense_attn_workspace_size.restype = ctypes.c_size_t
    L.csa2_dense_attn_workspace_size.argtypes = [i32, i32, i32]
    L.csa2_dense_swa_attn.argtypes = [ctypes.POINTER(KV), ctypes.POINTER(Rows), P, ctypes.c_int, i32, P, P, i64, P, P,
                                      P, f32, P, P, P, ctypes.c_size_t, P]
    L.csa2_synth_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint32, i64, i64, ctypes.c_int, P, P]
    L.csa2_synth_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint32, i64, i64, P, P]
    L.csa2_synth_boost.argtypes = [ctypes.c_uint64, ctypes.c_uint32, i64, i64, i32, P, P]
    L.csa2_stream_xor.argtypes = [P, i64, P, P]
    for name in EXPORTS:
        if name not in ("csa2_abi_version", "csa2_status_str", "csa2_last_error", "csa2_attn_workspace_size",
                        "csa2_select_topk_workspace", "csa2_dense_attn_workspace_size"):
            getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(fn, status):
    if status != 0:
        L = lib()
        raise Csa2Error(fn, status, (L.csa2_last_error() or b"").decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype(t):
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def make_kv(main_codes=None, main_scales=None, idx_codes=None, idx_scales=None, n_slots=0,
            page_entries=0, page_table=None, req_stride=0):
    """Host descriptor of a KV cache.  It keeps references to the tensors whose
    device pointers it holds, so they live as long as the descriptor."""
    max_pages = 0 if page_table is None else int(page_table.shape[-1])
    kv = KV(_ptr(main_codes), _ptr(main_scales), _ptr(idx_codes), _ptr(idx_scales), int(n_slots),
            int(page_entries), max_pages, _ptr(page_table), int(req_stride))
    kv._refs = (main_codes, main_scales, idx_codes, idx_scales, page_table)
    return kv


def make_rows(req, n_vis, max_vis):
    """Host descriptor of the query rows (keeps its tensors alive).  `req` may
    be None for csa2_index_score_shared, which takes the request as a value."""
    rows = Rows(_ptr(req), _ptr(n_vis), int(n_vis.shape[0]), int(max_vis))
    rows._refs = (req, n_vis)
    return rows


def _rstride(t) -> int:
    """Elements between consecutive rows of a 2-D (or wider) tensor; a tensor
    with one row may carry any stride on that axis, so its row length is used."""
    if t.dim() >= 2 and t.shape[0] == 1:
        return int(t[0].numel())
    return int(t.stride(0))


# ------------------------------------------------------------------ entry points
def abi_version() -> int:
    return lib().csa2_abi_version()


def csa2_pack_kv(kind, src, codes, scales, slots=None, stream=None):
    n = int(src.shape[0])
    _check("csa2_pack_kv", lib().csa2_pack_kv(kind, _ptr(src), _dtype(src), n, _rstride(src),
                                             _ptr(codes), _ptr(scales), _ptr(slots), _stream(stream)))


def csa2_compress_pack(kind, m, ca, za, ba, codes, scales, cb=None, zb=None, bb=None, norm_weight=None,
                       eps=1e-6, rope=True, pos0=0, values=None, slots=None, stream=None):
    """Compressed entries of the fp32 token streams (ca, za [n_tok, width];
    overlapping if cb, zb, bb are given), RMSNorm (if norm_weight), RoPE on
    the last 64 channels (if rope), packed to kind (MAIN_FP4 width 512 or
    INDEX_MXFP4 width 128) at slots; `values` receives the packed fp32 values."""
    st = CompressStreams(_ptr(ca), _ptr(za), _ptr(cb), _ptr(zb), _ptr(ba), _ptr(bb), int(ca.shape[0]),
                         _rstride(ca), int(m))
    _check("csa2_compress_pack", lib().csa2_compress_pack(
        int(kind), ctypes.byref(st), _ptr(norm_weight), float(eps), int(bool(rope)), int(pos0), _ptr(values),
        _ptr(codes), _ptr(scales), _ptr(slots), _stream(stream)))


def csa2_index_score(kv, rows, q_idx, w, scores=None, block_max=None, pool_blocks=None, pool_count=None,
                     stream=None):
    Hi = int(q_idx.shape[1])
    _check("csa2_index_score", lib().csa2_index_score(
        ctypes.byref(kv), ctypes.byref(rows), _ptr(q_idx), _dtype(q_idx), Hi, _ptr(w),
        _ptr(pool_blocks), 0 if pool_blocks is None else _rstride(pool_blocks), _ptr(pool_count),
        _ptr(scores), 0 if scores is None else _rstride(scores),
        _ptr(block_max), 0 if block_max is None else _rstride(block_max), _stream(stream)))


def csa2_index_score_shared(kv, rows, req, q_idx, w, scores=None, block_max=None, stream=None):
    """Full scan for query rows that all belong to request `req` (chunked
    prefill): each key tile is loaded once per 16 rows.  Same outputs as
    csa2_index_score's full scan."""
    Hi = int(q_idx.shape[1])
    _check("csa2_index_score_shared", lib().csa2_index_score_shared(
        ctypes.byref(kv), ctypes.byref(rows), int(req), _ptr(q_idx), _dtype(q_idx), Hi, _ptr(w),
        _ptr(scores), 0 if scores is None else _rstride(scores),
        _ptr(block_max), 0 if block_max is None else _rstride(block_max), _stream(stream)))


def csa2_select_topk_workspace(n_rows, max_cols, k) -> int:
    return int(lib().csa2_select_topk_workspace(int(n_rows), int(max_cols), int(k)))


def csa2_select_topk(keys, k, out_ids, out_count, n_cols=None, cols_mul=1, cols_div=1, pool_blocks=None,
                     keys_by_id=False, max_cols=None, ids=None, workspace=None, stream=None):
    """Row-wise top-k; `ids` (int32 [rows, >= max_cols], ascending per row)
    gives each column its id, else the column index or its pool position."""
    n_rows = int(out_ids.shape[0])
    if max_cols is None:
        max_cols = int(keys.shape[1]) if not keys_by_id else 8 * int(pool_blocks.shape[1])
    _check("csa2_select_topk", lib().csa2_select_topk(
        _ptr(keys), _rstride(keys), _ptr(ids), 0 if ids is None else _rstride(ids), _ptr(n_cols), cols_mul,
        cols_div, _ptr(pool_blocks), 0 if pool_blocks is None else _rstride(pool_blocks), int(bool(keys_by_id)),
        n_rows, int(max_cols), int(k), _ptr(out_ids), _rstride(out_ids), _ptr(out_count), *_ws(workspace),
        _stream(stream)))


def csa2_select_full(block_max, scores, n_vis, max_vis, pool, pool_count, idx, idx_count, n_pool_blocks=2048,
                     k=512, stream=None):
    """The Full layer's pool (top n_pool_blocks blocks by maximum) and its
    top-k positions, in one pass per row."""
    n_rows = int(pool.shape[0])
    _check("csa2_select_full", lib().csa2_select_full(
        _ptr(block_max), _rstride(block_max), _ptr(scores), _rstride(scores), _ptr(n_vis), n_rows, int(max_vis),
        int(n_pool_blocks), int(k), _ptr(pool), _rstride(pool), _ptr(pool_count), _ptr(idx), _rstride(idx),
        _ptr(idx_count), _stream(stream)))


def csa2_attn_workspace_size(n_rows, n_heads) -> int:
    return int(lib().csa2_attn_workspace_size(int(n_rows), int(n_heads)))


def _ws(workspace):
    return (None, 0) if workspace is None else (_ptr(workspace), int(workspace.numel() * workspace.element_size()))


def csa2_sparse_attn(kv, rows, q, idx, idx_count, softmax_scale, o_partial, lse, workspace=None, stream=None):
    H = int(q.shape[1])
    _check("csa2_sparse_attn", lib().csa2_sparse_attn(
        ctypes.byref(kv), ctypes.byref(rows), _ptr(q), _dtype(q), H, _ptr(idx), _rstride(idx),
        _ptr(idx_count), float(softmax_scale), _ptr(o_partial), _ptr(lse), *_ws(workspace),
        _stream(stream)))


def csa2_swa_merge(swa_codes, swa_scales, swa_first, swa_count, q, softmax_scale, out, sink=None,
                   o_partial=None, lse=None, workspace=None, stream=None):
    n_rows, H = int(q.shape[0]), int(q.shape[1])
    _check("csa2_swa_merge", lib().csa2_swa_merge(
        _ptr(swa_codes), _ptr(swa_scales), int(swa_codes.shape[0]), _ptr(swa_first), _ptr(swa_count), n_rows,
        _ptr(q), _dtype(q), H, float(softmax_scale), _ptr(sink), _ptr(o_partial), _ptr(lse), _ptr(out),
        *_ws(workspace), _stream(stream)))


def csa2_sparse_swa_attn(kv, rows, q, idx, idx_count, swa_codes, swa_scales, swa_first, swa_count, softmax_scale,
                         out, sink=None, lse=None, workspace=None, stream=None):
    H = int(q.shape[1])
    _check("csa2_sparse_swa_attn", lib().csa2_sparse_swa_attn(
        ctypes.byref(kv), ctypes.byref(rows), _ptr(q), _dtype(q), H, _ptr(idx), _rstride(idx),
        _ptr(idx_count), _ptr(swa_codes), _ptr(swa_scales), int(swa_codes.shape[0]), _ptr(swa_first),
        _ptr(swa_count), _ptr(sink), float(softmax_scale), _ptr(out), _ptr(lse),
        *_ws(workspace), _stream(stream)))


def csa2_sparse_swa_attn_noalloc(kv, rows, q, idx, idx_count, swa_codes, swa_scales, swa_first, swa_count,
                                 softmax_scale, out, sink=None, lse=None, stream=None):
    """csa2_sparse_swa_attn without a workspace: the split pass uses the
    library's own per-GPU scratch (calls overlapping on one GPU race)."""
    H = int(q.shape[1])
    _check("csa2_sparse_swa_attn_noalloc", lib().csa2_sparse_swa_attn_noalloc(
        ctypes.byref(kv), ctypes.byref(rows), _ptr(q), _dtype(q), H, _ptr(idx), _rstride(idx),
        _ptr(idx_count), _ptr(swa_codes), _ptr(swa_scales), int(swa_codes.shape[0]), _ptr(swa_first),
        _ptr(swa_count), _ptr(sink), float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream)))


def csa2_dense_attn_workspace_size(n_rows, n_heads, max_vis) -> int:
    return int(lib().csa2_dense_attn_workspace_size(int(n_rows), int(n_heads), int(max_vis)))


def csa2_dense_swa_attn(kv, rows, q, softmax_scale, out, swa_codes=None, swa_scales=None, swa_first=None,
                        swa_count=None, sink=None, lse=None, workspace=None, stream=None):
    """Attention over every visible entry of each row (the heavily
    compressed branch), jointly with the window (optional) and the sink."""
    H = int(q.shape[1])
    _check("csa2_dense_swa_attn", lib().csa2_dense_swa_attn(
        ctypes.byref(kv), ctypes.byref(rows), _ptr(q), _dtype(q), H, _ptr(swa_codes), _ptr(swa_scales),
        0 if swa_codes is None else int(swa_codes.shape[0]), _ptr(swa_first), _ptr(swa_count), _ptr(sink),
        float(softmax_scale), _ptr(out), _ptr(lse), *_ws(workspace), _stream(stream)))


def csa2_synth_normal(seed, tensor_id, first, out, stream=None):
    n = int(out.numel())
    _check("csa2_synth_normal", lib().csa2_synth_normal(int(seed), int(tensor_id), int(first), n,
                                                        _dtype(out), _ptr(out), _stream(stream)))


STREAM_XOR_WORDS = 1024


def csa2_stream_xor(buf, out, stream=None):
    """Streaming read of `buf` (device tensor, contiguous, 16-B aligned, size a multiple of 16 B): out[g]
    (a 32-bit device tensor of STREAM_XOR_WORDS elements) receives the XOR of the words workgroup g read."""
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    if out.numel() * out.element_size() < 4 * STREAM_XOR_WORDS:
        raise ValueError(f"out must hold {STREAM_XOR_WORDS} 32-bit words")
    _check("csa2_stream_xor", lib().csa2_stream_xor(_ptr(buf), int(buf.numel() * buf.element_size()), _ptr(out),
                                                    _stream(stream)))


def csa2_synth_uniform(seed, tensor_id, first, out, stream=None):
    _check("csa2_synth_uniform", lib().csa2_synth_uniform(int(seed), int(tensor_id), int(first),
                                                          int(out.numel()), _ptr(out), _stream(stream)))


def csa2_synth_boost(seed, tensor_id, first_pos, x, stream=None):
    _check("csa2_synth_boost", lib().csa2_synth_boost(int(seed), int(tensor_id), int(first_pos),
                                                      int(x.shape[0]), int(x.shape[1]), _ptr(x), _stream(stream)))
