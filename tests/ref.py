"""Oracle-side reference of one query row of a workload (tests only).

Draws the row's inputs with the host generator (synth), packs them with the
oracle's packers and runs the oracle's steps.  Nothing here comes from the
HIP path.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth
from synth.configs import Config

SIGMA = 512 ** -0.5


def f32(bits):
    return synth.bf16_bits_to_f32(bits)


class RowRef:
    def __init__(self, cfg: Config, row: int, layer: int = 0):
        self.cfg, self.row, self.layer = cfg, row, layer
        off = 16 * layer
        s = cfg.seed
        if cfg.mode == "prefill":
            t = cfg.prefill_tokens - cfg.prefill_rows + row
            self.req = 0
            self.n_vis = t // cfg.tokens_per_entry
            self.swa_first = row
        else:
            self.req = row
            self.n_vis = int(cfg.lens[row])
            self.swa_first = row * cfg.window
        self.base = int(cfg.req_base[self.req])
        H, Hi = cfg.heads, cfg.idx_heads
        self.q = f32(synth.normal_bf16(s, synth.T_Q + off, (H, 512), offset=row * H * 512))
        self.q_idx = f32(synth.normal_bf16(s, synth.T_QIDX + off, (Hi, 128), offset=row * Hi * 128))
        self.w = synth.uniform(s, synth.T_W + off, np.arange(row * Hi, row * Hi + Hi, dtype=np.uint64))
        self.qc, self.qs = oracle.quant_query(self.q_idx)
        # per-head sink logits of the layer (workloads that use one)
        self.sink = (f32(synth.normal_bf16(s, synth.T_SINK + off, (H,))) if cfg.extra.get("sink") else None)

    # ---------------------------------------------------------------- inputs
    def index_keys(self, pos):
        logical = self.base + np.asarray(pos, np.int64)
        x = f32(synth.normal_bf16_rows(self.cfg.seed, synth.T_IDXKEY, logical, 128))
        if self.cfg.boost:
            x = np.where(synth.boost_mask(self.cfg.seed, logical)[:, None], x * np.float32(3), x).astype(np.float32)
        return x

    def packed_index(self, pos):
        return oracle.pack_index(self.index_keys(pos))

    def latent(self, pos):
        logical = self.base + np.asarray(pos, np.int64)
        return f32(synth.normal_bf16_rows(self.cfg.seed, synth.T_LATENT, logical, 512))

    def swa(self):
        ids = self.swa_first + np.arange(self.cfg.window, dtype=np.int64)
        return f32(synth.normal_bf16_rows(self.cfg.seed, synth.T_SWA + 16 * self.layer, ids, 512))

    # ---------------------------------------------------------------- steps
    def scores_at(self, pos, chunk: int = 1 << 15):
        """Oracle scores of the given positions; long lists are split into
        chunks scored on a thread pool (each chunk is independent)."""
        pos = np.asarray(pos, np.int64)

        def one(p):
            kc, ks = self.packed_index(p)
            return oracle.index_score(self.qc, self.qs, self.w, kc, ks)

        if len(pos) <= chunk:
            return one(pos)
        parts = [pos[i:i + chunk] for i in range(0, len(pos), chunk)]
        return np.concatenate(oracle.map_rows(one, parts))

    def full_scores(self):
        return self.scores_at(np.arange(self.n_vis))

    def select_full(self, scores):
        return oracle.full_select(scores)

    def select_pool(self, pool):
        pos = oracle.pool_positions(pool, self.n_vis)
        sc = self.scores_at(pos)
        return pos, sc, oracle.topk(sc, 512, ids=pos)

    def select_prefill(self, scores):
        return oracle.topk(scores, 512)

    def attend_dense(self):
        """Every visible entry of the row (the heavily compressed branch),
        the window and the layer's sink."""
        _, _, o = self.attend(np.arange(self.n_vis, dtype=np.int64), sink=self.sink)
        return o

    def attend(self, idx, sink=None):
        kc, ks = oracle.pack_main(self.latent(idx))
        K = oracle.dequant_main(kc, ks)
        wc, wsc = oracle.pack_swa(self.swa())
        W = oracle.dequant_swa(wc, wsc)
        o_p, lse_p = oracle.attention(self.q, K, None, sigma=SIGMA)
        o, lse = oracle.attention(self.q, K, W, sink=sink, sigma=SIGMA)
        return o_p, lse_p, o
