"""CPU oracle of the CSA2 decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never does, and the two
share no code: the arithmetic lives in ``csa2_oracle.c`` (plain scalar C, fp64
attention, exact integer indexer dot products), this module only marshals
numpy arrays and strings the per-row steps together in the order the pages
give them.

Sources (by page title and section):
  * "DeepSeek-V4: Towards Highly Efficient Million-Token Context
    Intelligence" (Korean translation page), section 2.3.1: index score
    I_{t,s} = sum_h w_h ReLU(q_h . K_s), top-k selection, shared-KV MQA where
    each selected entry is key and value; section 2.3.3: sliding-window
    branch attended together with the selected entries, attention sink;
    section 2.3.4: indexer attention computed in FP4.
  * "DeepSeek V4.1 Flash architecture analysis" (plaidlabs page), sections on
    the hierarchical sparse indexer (the first Full layer scores every
    position, keeps up to 2,048 groups of 8 by their maximum, Reindex layers
    choose their own top-512 inside that pool) and "890 bytes/token" (entry
    formats: 512 x E2M1 + 32 E4M3 scales = 288 B; 128 x E2M1 + 4 E8M0 = 68 B).
  * "KV cache diet" page (ithotfix), figure 2 and the "890 ... 10,324"
    section: layer roles, byte arithmetic, SWA kept in FP8.
  * MLA article (huny.dev), section 4: matrix absorption -- attention over the
    latent with the absorbed query equals the up-projected attention.

Every function here has a pin in ``tests/test_oracle_*.py`` (see the module
docstrings there); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

N_POOL_BLOCKS = 2048     # candidate_topk_blocks
BLOCK = 8                # candidate_block_size
INDEX_TOPK = 512         # index_topk
WINDOW = 128             # sliding window


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (in place)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e2m1_value.argtypes = [ctypes.c_uint]
        L.orc_e2m1_encode.restype = ctypes.c_uint
        L.orc_e2m1_encode.argtypes = [ctypes.c_double]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_uint]
        L.orc_e4m3_encode.restype = ctypes.c_uint
        L.orc_e4m3_encode.argtypes = [ctypes.c_double]
        L.orc_e8m0_value.restype = ctypes.c_double
        L.orc_e8m0_value.argtypes = [ctypes.c_uint]
        for name in ("orc_pack_main", "orc_pack_index", "orc_pack_swa",
                     "orc_dequant_main", "orc_dequant_index", "orc_dequant_swa"):
            getattr(L, name).restype = None
        L.orc_pack_main.argtypes = [P, i64, P, P]
        L.orc_pack_index.argtypes = [P, i64, P, P]
        L.orc_pack_swa.argtypes = [P, i64, P, P]
        L.orc_dequant_main.argtypes = [P, P, i64, P]
        L.orc_dequant_index.argtypes = [P, P, i64, P]
        L.orc_dequant_swa.argtypes = [P, P, i64, P]
        L.orc_round_pow2_sum.restype = ctypes.c_float
        L.orc_round_pow2_sum.argtypes = [P, P, ctypes.c_int]
        L.orc_head_dot.restype = ctypes.c_float
        L.orc_head_dot.argtypes = [P, P, P, P]
        L.orc_index_score.restype = None
        L.orc_index_score.argtypes = [P, P, P, ctypes.c_int, P, P, i64, P]
        L.orc_block_max.restype = None
        L.orc_block_max.argtypes = [P, i64, P]
        L.orc_topk.restype = i64
        L.orc_topk.argtypes = [P, P, i64, i64, P]
        L.orc_attention.restype = None
        L.orc_attention.argtypes = [P, ctypes.c_int, ctypes.c_int, P, i64, P, i64, P,
                                    ctypes.c_double, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- codecs
def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(code)


def e2m1_encode(x: float) -> int:
    return lib().orc_e2m1_encode(float(x))


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(code)


def e4m3_encode(x: float) -> int:
    return lib().orc_e4m3_encode(float(x))


def e8m0_value(code: int) -> float:
    return lib().orc_e8m0_value(code)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- packing
def pack_main(x: np.ndarray):
    """[n, 512] fp32 -> (codes [n, 256] u8, scales [n, 32] u8)."""
    x = _c(x, np.float32).reshape(-1, 512)
    n = x.shape[0]
    codes = np.zeros((n, 256), np.uint8)
    scales = np.zeros((n, 32), np.uint8)
    lib().orc_pack_main(_p(x), n, _p(codes), _p(scales))
    return codes, scales


def pack_index(x: np.ndarray):
    """[n, 128] fp32 -> (codes [n, 64], scales [n, 4])."""
    x = _c(x, np.float32).reshape(-1, 128)
    n = x.shape[0]
    codes = np.zeros((n, 64), np.uint8)
    scales = np.zeros((n, 4), np.uint8)
    lib().orc_pack_index(_p(x), n, _p(codes), _p(scales))
    return codes, scales


def pack_swa(x: np.ndarray):
    """[n, 512] fp32 -> (codes [n, 512], scales [n, 32])."""
    x = _c(x, np.float32).reshape(-1, 512)
    n = x.shape[0]
    codes = np.zeros((n, 512), np.uint8)
    scales = np.zeros((n, 32), np.uint8)
    lib().orc_pack_swa(_p(x), n, _p(codes), _p(scales))
    return codes, scales


def dequant_main(codes, scales):
    codes = _c(codes, np.uint8).reshape(-1, 256)
    scales = _c(scales, np.uint8).reshape(-1, 32)
    out = np.zeros((codes.shape[0], 512), np.float32)
    lib().orc_dequant_main(_p(codes), _p(scales), codes.shape[0], _p(out))
    return out


def dequant_index(codes, scales):
    codes = _c(codes, np.uint8).reshape(-1, 64)
    scales = _c(scales, np.uint8).reshape(-1, 4)
    out = np.zeros((codes.shape[0], 128), np.float32)
    lib().orc_dequant_index(_p(codes), _p(scales), codes.shape[0], _p(out))
    return out


def dequant_swa(codes, scales):
    codes = _c(codes, np.uint8).reshape(-1, 512)
    scales = _c(scales, np.uint8).reshape(-1, 32)
    out = np.zeros((codes.shape[0], 512), np.float32)
    lib().orc_dequant_swa(_p(codes), _p(scales), codes.shape[0], _p(out))
    return out


# ---------------------------------------------------------------- indexer
def round_pow2_sum(S, E) -> float:
    S = _c(S, np.int64)
    E = _c(E, np.int32)
    return float(lib().orc_round_pow2_sum(_p(S), _p(E), len(S)))


def head_dot(qc, qs, kc, ks) -> float:
    qc, qs, kc, ks = (_c(a, np.uint8) for a in (qc, qs, kc, ks))
    return float(lib().orc_head_dot(_p(qc), _p(qs), _p(kc), _p(ks)))


def index_score(q_codes, q_scales, w, k_codes, k_scales) -> np.ndarray:
    """Scores of n MXFP4 keys for one row.  q_codes [Hi, 64], q_scales [Hi, 4],
    w [Hi] fp32, k_codes [n, 64], k_scales [n, 4] -> fp32 [n]."""
    qc = _c(q_codes, np.uint8).reshape(-1, 64)
    qs = _c(q_scales, np.uint8).reshape(-1, 4)
    w = _c(w, np.float32).reshape(-1)
    kc = _c(k_codes, np.uint8).reshape(-1, 64)
    ks = _c(k_scales, np.uint8).reshape(-1, 4)
    assert qc.shape[0] == qs.shape[0] == w.shape[0] and kc.shape[0] == ks.shape[0]
    out = np.zeros(kc.shape[0], np.float32)
    lib().orc_index_score(_p(qc), _p(qs), _p(w), qc.shape[0], _p(kc), _p(ks), kc.shape[0], _p(out))
    return out


def block_max(scores) -> np.ndarray:
    s = _c(scores, np.float32).reshape(-1)
    out = np.zeros((len(s) + BLOCK - 1) // BLOCK, np.float32)
    lib().orc_block_max(_p(s), len(s), _p(out))
    return out


def topk(keys, k: int, ids=None) -> np.ndarray:
    """ids of the min(k, n) items first in (key desc, id asc), ascending."""
    keys = _c(keys, np.float32).reshape(-1)
    ids_a = None if ids is None else _c(ids, np.int32).reshape(-1)
    out = np.zeros(max(min(k, len(keys)), 0), np.int32)
    m = lib().orc_topk(_p(keys), _p(ids_a), len(keys), k, _p(out))
    if m < 0:
        raise MemoryError("oracle top-k")
    return out[:m]


# ---------------------------------------------------------------- attention
def attention(q, K=None, W=None, sink=None, sigma: float = 512 ** -0.5):
    """q [H, C] fp32, K [n, C], W [m, C] dequantised entries -> (o [H, C], lse [H])."""
    q = _c(q, np.float32)
    H, C = q.shape
    K = np.zeros((0, C), np.float32) if K is None else _c(K, np.float32).reshape(-1, C)
    W = np.zeros((0, C), np.float32) if W is None else _c(W, np.float32).reshape(-1, C)
    s = None if sink is None else _c(sink, np.float32).reshape(H)
    o = np.zeros((H, C), np.float32)
    lse = np.zeros(H, np.float32)
    lib().orc_attention(_p(q), H, C, _p(K), K.shape[0], _p(W), W.shape[0], _p(s),
                        float(sigma), _p(o), _p(lse))
    return o, lse


# ---------------------------------------------------------------- the steps
def pool_positions(pool_blocks, n_vis: int) -> np.ndarray:
    """Positions 8b .. 8b+7 (below n_vis) of each pool block, ascending."""
    b = np.asarray(pool_blocks, np.int64).reshape(-1, 1)
    pos = (BLOCK * b + np.arange(BLOCK).reshape(1, -1)).reshape(-1)
    return pos[pos < n_vis].astype(np.int32)


def full_select(scores, n_pool: int = N_POOL_BLOCKS, k: int = INDEX_TOPK):
    """First Full layer: pool = top n_pool blocks by block max; idx = top-k
    positions inside the pool.  Returns (pool_blocks, idx), both ascending."""
    scores = _c(scores, np.float32).reshape(-1)
    pool = topk(block_max(scores), n_pool)
    pos = pool_positions(pool, len(scores))
    idx = topk(scores[pos], k, ids=pos)
    return pool, idx


def quant_query(q_idx):
    """Indexer query [Hi, 128] fp32 -> MXFP4 (codes [Hi, 64], scales [Hi, 4])."""
    return pack_index(q_idx)


def default_threads() -> int:
    """Host threads for the oracle: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def map_rows(fn, items, threads: int | None = None):
    """Run ``fn`` over independent rows on a thread pool (the C calls release
    the GIL); returns the results in order."""
    threads = threads or default_threads()
    if threads <= 1 or len(items) <= 1:
        return [fn(it) for it in items]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, items))
