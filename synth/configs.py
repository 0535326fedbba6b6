"""The synthetic workloads (shapes, seeds, structure) -- data only.

Element numbering shared by every consumer (host generator, GPU generator,
oracle): a cache entry has a *logical* id ``req_base[req] + pos`` (requests
laid end to end); element c of a tensor row r is element ``r * width + c`` of
that tensor's stream.  Per-layer streams add 16 * layer to the tensor id.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import ragged_lengths


@dataclass
class Config:
    name: str
    seed: int
    n_req: int
    heads: int = 64
    idx_heads: int = 8
    mode: str = "full"            # "full" | "reindex" | "prefill" | "mixed" | "dense" | "csa"
    ctx: int = 0                  # entries per request (uniform contexts)
    lengths: np.ndarray | None = None   # ragged contexts (entries)
    page_entries: int = 0         # 0 = contiguous
    reindex_layers: int = 0
    boost: bool = False
    prefill_rows: int = 0         # chunked prefill: query rows (tokens)
    prefill_tokens: int = 0       # total tokens of the prefill context
    tokens_per_entry: int = 1
    window: int = 128
    description: str = ""
    extra: dict = field(default_factory=dict)
    layer_roles: tuple | None = None   # per layer: "full" | "reindex" | "reuse" (None: from mode)

    @property
    def roles(self) -> tuple:
        """The role of each layer of a step: a Full layer scores every
        position and builds the pool, a Reindex layer re-scores the pool with
        its own indexer query, a Reuse layer attends with its own query over
        the positions the last Full or Reindex layer chose."""
        if self.layer_roles is not None:
            return tuple(self.layer_roles)
        if self.mode == "reindex":
            return ("reindex",)
        if self.mode == "prefill":
            return ("prefill",)
        if self.mode == "dense":
            return ("dense",)
        return ("full",) + ("reindex",) * self.reindex_layers

    @property
    def lens(self) -> np.ndarray:
        if self.lengths is not None:
            return np.asarray(self.lengths, np.int64)
        return np.full(self.n_req, self.ctx, np.int64)

    @property
    def total_entries(self) -> int:
        return int(self.lens.sum())

    @property
    def req_base(self) -> np.ndarray:
        L = self.lens
        return np.concatenate([[0], np.cumsum(L)[:-1]]).astype(np.int64)


def tiny_full_decode(**kw) -> Config:
    return Config("tiny_full_decode_4k", seed=0, n_req=1, heads=16, ctx=4096, mode="full",
                  description="1 request, 4,096 cached entries, 16 heads, Full layer", **kw)


def full_decode_128k(**kw) -> Config:
    return Config("full_decode_16x128k", seed=1, n_req=16, heads=64, ctx=131072, mode="full",
                  description="16 requests x 131,072 entries, 64 heads, Full layer", **kw)


def reindex_decode_1m(**kw) -> Config:
    return Config("reindex_decode_64x1m", seed=2, n_req=64, heads=64, ctx=1048576, mode="reindex",
                  boost=True, description="64 requests x 1,048,576 entries, given 2,048-block pools, "
                  "5% of indexer keys x3, 64 heads, Reindex layer", **kw)


def chunked_prefill_256k(**kw) -> Config:
    return Config("chunked_prefill_4096x131k", seed=3, n_req=1, heads=64, ctx=131072, mode="prefill",
                  prefill_rows=4096, prefill_tokens=262144, tokens_per_entry=2,
                  description="262,144 tokens at 2 per entry (131,072 entries); the last 4,096 tokens "
                  "as causal query rows, 64 heads", **kw)


def mixed_serving(**kw) -> Config:
    seed = 4
    return Config("mixed_serving_256req", seed=seed, n_req=256, heads=64, mode="mixed",
                  lengths=ragged_lengths(seed, 256), page_entries=64, reindex_layers=4,
                  description="256 requests, log-uniform contexts in [4,096, 1,048,576), 64-entry pages "
                  "in a random page order, 1 Full + 4 Reindex layers, 64 heads", **kw)


def v4_csa_decode_1m(**kw) -> Config:
    # the compressed sparse attention of the V4 hybrid ('DeepSeek-V4' page,
    # section 2.3.1 and the model setup of section 4.2.1: 4 tokens per entry,
    # 64 indexer heads of 128 channels, top-512 over every visible compressed
    # entry, no block pool), with the window and a per-head sink (2.3.3)
    return Config("v4_csa_decode_16x1m", seed=8, n_req=16, heads=64, idx_heads=64, ctx=262144, mode="csa",
                  tokens_per_entry=4, extra={"sink": True},
                  description="16 requests x 1,048,576 tokens at 4 per entry (262,144 entries), 64 indexer heads, "
                  "top-512 over all entries, 64 heads, window 128 + sink", **kw)


def hca_decode_1m(**kw) -> Config:
    # the heavily compressed branch of the V4 hybrid attention ('DeepSeek-V4'
    # page, section 2.3.2): every 128 tokens of a 1,048,576-token context
    # compressed into one entry (8,192 per request), attended densely with the
    # sliding window and a per-head sink (section 2.3.3)
    return Config("hca_decode_16x1m", seed=6, n_req=16, heads=64, ctx=8192, mode="dense", tokens_per_entry=128,
                  extra={"sink": True}, description="16 requests x 1,048,576 tokens at 128 per entry (8,192 "
                  "entries), 64 heads, dense attention over every entry + window 128 + sink", **kw)


def decoder_stack_128k(**kw) -> Config:
    # the decoder's 20 CSA2 layers: one Full or Reindex layer, then three
    # Reuse layers, four times over ('KV cache diet' page, figure 2 and the
    # layer roles; V4.1 Flash architecture page, "Global KV is built in four
    # places")
    roles = tuple("full" if i == 0 else "reindex" if i % 4 == 0 else "reuse" for i in range(20))
    return Config("decoder_stack_16x128k", seed=5, n_req=16, heads=64, ctx=131072, mode="full",
                  layer_roles=roles, description="16 requests x 131,072 entries, 64 heads, the decoder's 20 "
                  "layers: 1 Full, 4 Reindex, 15 Reuse", **kw)


ALL = {
    "c0": tiny_full_decode,
    "c1": full_decode_128k,
    "c2": reindex_decode_1m,
    "c3": chunked_prefill_256k,
    "c4": mixed_serving,
    "stack": decoder_stack_128k,
    "hca": hca_decode_1m,
    "v4csa": v4_csa_decode_1m,
}
