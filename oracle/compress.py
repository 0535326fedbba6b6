"""CPU oracle of the write path that fills the compressed cache -- TEST
INFRASTRUCTURE ONLY (tests/, the smoke check and the bench's CPU leg may use
it; the HIP library never does and shares no code with it).

Plain numpy in fp64, step by step as the pages give it:

* 'DeepSeek-V4' page, section 2.3.1, "compressed key-value entries": two
  projected streams C^a, C^b (values) and Z^a, Z^b (compression logits) of
  shape [n, c], learnable positional biases B^a, B^b of shape [m, c].  Entry
  i is built from the m tokens of block i (the a stream) and the m tokens of
  block i - 1 (the b stream): per channel, a softmax over those 2m logits
  Z + B (jointly over both streams), then the weighted sum of the matching
  C rows.  For i = 0 the b part is padding: logits -inf, values 0.
* same page, section 2.3.2 (heavily compressed attention): one stream C, Z,
  bias B of shape [m', c], blocks of m' tokens, no overlap.
* same page, section 2.3.3: an RMSNorm of the compressed entry (one head)
  before the core attention, and a rotary position embedding on the last 64
  channels of every KV entry.  Readings where the page is silent: RMSNorm
  y = x / sqrt(mean(x^2) + eps) * weight; RoPE rotates consecutive channel
  pairs (2j, 2j+1) of the last 64 channels by pos * base^(-2j/64) with base
  10,000; compressed entry i sits at token position pos0 + m * i (the first
  token of its own block).
* 'KV cache diet' page, "890 ... 10,324": quantisation comes after RoPE, so
  the packed entry is the rotated one (the packers of oracle/__init__.py).
* The indexer keys take "the same compression operation" (section 2.3.1,
  lightning indexer) and no norm or rotation is stated for them: compression
  only.
"""
from __future__ import annotations

import numpy as np

ROPE_DIMS = 64
ROPE_BASE = 10000.0


def _softmax_rows(logits):
    """Softmax over axis 0 (the tokens of one entry), per channel; -inf rows
    get weight 0."""
    mx = np.max(logits, axis=0, keepdims=True)
    e = np.exp(logits - mx)
    return e / np.sum(e, axis=0, keepdims=True)


def compress_overlap(ca, za, cb, zb, ba, bb, m: int) -> np.ndarray:
    """Gated overlapping compression: [n, c] streams -> [n // m, c] entries
    (complete blocks only)."""
    ca, za, cb, zb = (np.asarray(x, np.float64) for x in (ca, za, cb, zb))
    ba, bb = np.asarray(ba, np.float64), np.asarray(bb, np.float64)
    n, c = ca.shape
    out = np.zeros((n // m, c))
    for i in range(n // m):
        la = za[m * i:m * (i + 1)] + ba
        va = ca[m * i:m * (i + 1)]
        if i == 0:
            lb = np.full((m, c), -np.inf)
            vb = np.zeros((m, c))
        else:
            lb = zb[m * (i - 1):m * i] + bb
            vb = cb[m * (i - 1):m * i]
        s = _softmax_rows(np.concatenate([la, lb], axis=0))
        out[i] = np.sum(s[:m] * va, axis=0) + np.sum(s[m:] * vb, axis=0)
    return out


def compress_block(cv, z, b, m: int) -> np.ndarray:
    """Non-overlapping compression of every m tokens (the heavily compressed
    branch): softmax over the block's m logits Z + B per channel, weighted
    sum of the block's values."""
    cv, z, b = (np.asarray(x, np.float64) for x in (cv, z, b))
    n, c = cv.shape
    out = np.zeros((n // m, c))
    for i in range(n // m):
        s = _softmax_rows(z[m * i:m * (i + 1)] + b)
        out[i] = np.sum(s * cv[m * i:m * (i + 1)], axis=0)
    return out


def rms_norm(x, weight, eps: float) -> np.ndarray:
    """Per entry (row): x / sqrt(mean(x^2) + eps) * weight."""
    x = np.asarray(x, np.float64)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x / r * np.asarray(weight, np.float64)


def rope_tail(x, pos, dims: int = ROPE_DIMS, base: float = ROPE_BASE) -> np.ndarray:
    """Rotate the last `dims` channels of each row: pair j = channels
    (c - dims + 2j, c - dims + 2j + 1) by the angle pos * base^(-2j/dims)."""
    x = np.array(x, np.float64, copy=True)
    pos = np.asarray(pos, np.float64).reshape(-1, 1)
    c = x.shape[-1]
    j = np.arange(dims // 2, dtype=np.float64)
    ang = pos * base ** (-2.0 * j / dims)
    cs, sn = np.cos(ang), np.sin(ang)
    x0 = x[:, c - dims::2].copy()
    x1 = x[:, c - dims + 1::2].copy()
    x[:, c - dims::2] = x0 * cs - x1 * sn
    x[:, c - dims + 1::2] = x0 * sn + x1 * cs
    return x


def write_entries(m: int, ca, za, ba, cb=None, zb=None, bb=None, norm_weight=None, eps: float = 1e-6,
                  rope: bool = True, pos0: int = 0) -> np.ndarray:
    """The values a compressed cache entry holds before quantisation:
    compression (overlapping if the b stream is given), then the RMSNorm (if
    a weight is given), then RoPE on the last 64 channels (if `rope`) at
    position pos0 + m * i.  fp64, [n // m, c]."""
    if cb is not None:
        e = compress_overlap(ca, za, cb, zb, ba, bb, m)
    else:
        e = compress_block(ca, za, ba, m)
    if norm_weight is not None:
        e = rms_norm(e, norm_weight, eps)
    if rope:
        e = rope_tail(e, pos0 + m * np.arange(e.shape[0]))
    return e
