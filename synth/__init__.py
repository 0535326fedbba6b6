"""Seeded synthetic inputs for the CSA2 decode path (numpy, host side).

This module only draws numbers: it holds none of the method's arithmetic (no
quantisation, scoring, selection or attention).  Both the HIP library's tests
and the CPU oracle take their inputs from here, and the HIP library carries its
own device implementation of the same counter-based generator (so that very
large caches can be drawn on the GPU) which is checked bit for bit against this
one.

Generator definition (counter based, so any element can be drawn on its own):

* ``mix64`` is the SplitMix64 output finaliser (Steele, Lea & Flood, "Fast
  splittable pseudorandom number generators", OOPSLA 2014; constants of
  Vigna's public-domain ``splitmix64.c``).
* A stream is named by ``(seed, tensor_id)``:
  ``base = mix64(seed * GAMMA + tensor_id)``.
* Word ``i`` of a stream is ``mix64(base + (i + 1) * GAMMA)`` (all arithmetic
  modulo 2**64), i.e. the i-th output of SplitMix64 seeded with ``base``.
* ``uniform(i) = (word(i) >> 40) * 2**-24``, exact in fp32, in [0, 1).
* ``normal(i)`` uses words ``3i, 3i+1, 3i+2``; each word gives four 16-bit
  fields (bits 0-15, 16-31, 32-47, 48-63); ``X = (sum of the 12 fields -
  393210) * 2**-16``.  This is an Irwin-Hall approximation of N(0, 1):
  exact in fp32, variance (2**32 - 1) / 2**32, bounded by 6.
* ``bf16`` values are the round-to-nearest-even bf16 of the fp32 value.
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# Tensor ids of the streams one decode layer draws from.  A layer offset of
# 16 * layer keeps the streams of stacked layers apart.
T_LATENT = 1      # 512-channel latent KV (packed to the FP4 main cache)
T_IDXKEY = 2      # 128-channel indexer keys (packed to MXFP4)
T_Q = 3           # attention query, 512 channels per head (bf16)
T_QIDX = 4        # indexer query, 128 channels per indexer head
T_W = 5           # indexer head weights, U(0, 1)
T_SWA = 6         # sliding-window KV, 512 channels (packed to FP8)
T_POOL = 7        # hash used to draw a given candidate pool
T_BOOST = 8       # hash used to pick boosted indexer keys
T_LEN = 9         # ragged context lengths
T_PAGE = 10       # page permutation
T_SINK = 11       # attention-sink logits (tests only)


def _u64(x):
    return np.asarray(x, dtype=np.uint64)


def mix64(z):
    z = _u64(z).copy()
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= _M1
        z ^= z >> np.uint64(27)
        z *= _M2
        z ^= z >> np.uint64(31)
    return z


def stream_base(seed: int, tensor_id: int) -> np.uint64:
    with np.errstate(over="ignore"):
        v = np.uint64(seed) * GAMMA + np.uint64(tensor_id)
    return mix64(v)[()]


def words(seed: int, tensor_id: int, idx) -> np.ndarray:
    """64-bit words ``idx`` (array of non-negative integers) of a stream."""
    base = stream_base(seed, tensor_id)
    i = _u64(idx)
    with np.errstate(over="ignore"):
        return mix64(base + (i + np.uint64(1)) * GAMMA)


def uniform(seed: int, tensor_id: int, idx) -> np.ndarray:
    w = words(seed, tensor_id, idx)
    return ((w >> np.uint64(40)).astype(np.float64) * 2.0 ** -24).astype(np.float32)


def normal(seed: int, tensor_id: int, idx) -> np.ndarray:
    """fp32 Irwin-Hall normals for element indices ``idx``."""
    base = stream_base(seed, tensor_id)
    flat = _u64(idx).reshape(-1)
    out = np.empty(flat.shape[0], np.float32)
    step = 1 << 16                      # chunks stay in cache
    with np.errstate(over="ignore"):
        for c0 in range(0, flat.shape[0], step):
            i3 = flat[c0:c0 + step] * np.uint64(3)
            tot = np.zeros(i3.shape[0], np.int64)
            for k in range(3):
                z = (i3 + np.uint64(k + 1)) * GAMMA
                z += base
                z ^= z >> np.uint64(30)
                z *= _M1
                z ^= z >> np.uint64(27)
                z *= _M2
                z ^= z >> np.uint64(31)
                # the four 16-bit fields of each word (their order does not matter)
                tot += z.view(np.uint16).reshape(-1, 4).astype(np.int64).sum(axis=1)
            out[c0:c0 + step] = (tot - 393210).astype(np.float64) * 2.0 ** -16
    return out.reshape(np.shape(idx))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, tensor_id: int, shape, offset: int = 0) -> np.ndarray:
    """bf16 bit patterns of N(0,1) draws for a dense tensor of ``shape``
    (element index = ``offset`` + row-major linear index)."""
    n = int(np.prod(shape))
    x = normal(seed, tensor_id, np.arange(offset, offset + n, dtype=np.uint64))
    return f32_to_bf16_bits(x).reshape(shape)


def normal_bf16_rows(seed: int, tensor_id: int, row_ids, width: int) -> np.ndarray:
    """bf16 bit patterns of rows ``row_ids`` of a [*, width] tensor."""
    r = _u64(row_ids).reshape(-1, 1)
    idx = r * np.uint64(width) + np.arange(width, dtype=np.uint64).reshape(1, -1)
    return f32_to_bf16_bits(normal(seed, tensor_id, idx)).reshape(len(r), width)


def uniform_f32(seed: int, tensor_id: int, shape, offset: int = 0) -> np.ndarray:
    n = int(np.prod(shape))
    return uniform(seed, tensor_id, np.arange(offset, offset + n, dtype=np.uint64)).reshape(shape)


def boost_mask(seed: int, positions) -> np.ndarray:
    """True for the ~5% of positions whose indexer keys are multiplied by 3
    (hash word below 0.05 * 2**64)."""
    w = words(seed, T_BOOST, _u64(positions))
    return w < np.uint64(int(0.05 * 2 ** 64))


def given_pool(seed: int, row: int, n_blocks_total: int, n_pool: int) -> np.ndarray:
    """A random set of ``n_pool`` distinct block ids out of ``n_blocks_total``,
    sorted ascending: the blocks with the smallest hash words (ties by id)."""
    idx = np.arange(n_blocks_total, dtype=np.uint64) + np.uint64(row) * np.uint64(n_blocks_total)
    h = words(seed, T_POOL, idx)
    order = np.lexsort((np.arange(n_blocks_total), h))
    return np.sort(order[:n_pool]).astype(np.int32)


def ragged_lengths(seed: int, n: int, lo: int = 4096, span_log2: int = 8) -> np.ndarray:
    """Context lengths ``floor(lo * 2**(span_log2 * U))``, U ~ U(0, 1): log-uniform
    on [lo, lo * 2**span_log2)."""
    u = uniform(seed, T_LEN, np.arange(n, dtype=np.uint64)).astype(np.float64)
    return np.floor(lo * np.exp2(span_log2 * u)).astype(np.int64)


def page_permutation(seed: int, n_pages: int) -> np.ndarray:
    """A random permutation of ``n_pages`` physical pages (sort by hash)."""
    h = words(seed, T_PAGE, np.arange(n_pages, dtype=np.uint64))
    return np.lexsort((np.arange(n_pages), h)).astype(np.int32)
