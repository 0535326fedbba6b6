"""Device-resident synthetic workloads and the decode step that runs them.

Builds the caches of a configuration (synth.configs) on the GPU with the
library's own generator and packer, then strings the five entry points
together as one step of the hot path:

  Full layer    csa2_index_score (full scan + block max)
                -> csa2_select_full (2,048 blocks, then 512 positions among them;
                   or the two csa2_select_topk calls)
                -> csa2_sparse_swa_attn (or csa2_sparse_attn -> csa2_swa_merge)
  Reindex layer csa2_index_score (pool) -> csa2_select_topk (512)
                -> csa2_sparse_swa_attn (or csa2_sparse_attn -> csa2_swa_merge)
  Reuse layer   csa2_sparse_swa_attn with the layer's own query and window over
                the positions the last Full or Reindex layer selected
  Dense layer   csa2_dense_swa_attn over every compressed entry (the heavily
                compressed branch of the V4 hybrid attention), window, sink

A whole step (every layer) can also be captured once per KV copy as a HIP
graph and replayed (``capture_graphs`` / ``replay``).

('DeepSeek V4.1 Flash architecture analysis' page, hierarchical sparse
indexer: the first Full layer scores every position and builds the pool that
later Reindex layers re-score, and a Reuse layer still attends with its own
query over the shared positions; 'KV cache diet' page, figure 2: layer roles.)
"""
from __future__ import annotations

import math

import numpy as np
import torch

import synth
from synth.configs import Config

from . import (BF16, F32, INDEX_MXFP4, MAIN_FP4, SWA_FP8, csa2_attn_workspace_size, csa2_dense_attn_workspace_size,
               csa2_dense_swa_attn, csa2_index_score, csa2_index_score_shared, csa2_pack_kv, csa2_select_full,
               csa2_select_topk, csa2_sparse_attn, csa2_sparse_swa_attn, csa2_swa_merge, csa2_synth_boost,
               csa2_synth_normal, csa2_synth_uniform, make_kv, make_rows)

GEN_CHUNK = 1 << 20   # entries generated per chunk


def _planes(n, kind, dev):
    cb, sb = {MAIN_FP4: (256, 32), INDEX_MXFP4: (64, 4), SWA_FP8: (512, 32)}[kind]
    return (torch.empty((n, cb), dtype=torch.uint8, device=dev),
            torch.empty((n, sb), dtype=torch.uint8, device=dev))


def _fill_packed(kind, seed, tensor, width, logical_first, n, codes, scales, slots=None, boost=False,
                 dev="cuda"):
    """Generate rows logical_first .. +n of stream (seed, tensor) and pack them.
    Row i goes to entry slots[i] (or to row i of codes/scales)."""
    for c0 in range(0, n, GEN_CHUNK):
        m = min(GEN_CHUNK, n - c0)
        buf = torch.empty((m, width), dtype=torch.float32 if boost else torch.bfloat16, device=dev)
        csa2_synth_normal(seed, tensor, (logical_first + c0) * width, buf)
        if boost:
            csa2_synth_boost(seed, synth.T_BOOST, logical_first + c0, buf)
        if slots is None:
            csa2_pack_kv(kind, buf, codes[c0:c0 + m], scales[c0:c0 + m])
        else:
            csa2_pack_kv(kind, buf, codes, scales, slots=slots[c0:c0 + m])
        del buf


def _padded_rows(n_rows: int, n: int, dev) -> torch.Tensor:
    """[n_rows][n] fp32 whose rows start on 64-B boundaries, so that the
    selection reads whole runs of block maxima with 16-B loads."""
    return torch.empty((n_rows, (n + 15) // 16 * 16), dtype=torch.float32, device=dev)[:, :n]


class Layer:
    """Per-layer query-side inputs and outputs of one step.  A Reuse layer
    (``source`` given) has no indexer inputs and reads the selection of its
    source layer."""

    def __init__(self, cfg: Config, n_rows: int, layer: int, swa_first_tok, dev, role: str = "full",
                 source: "Layer | None" = None):
        self.role = role
        self.index = layer
        H, Hi = cfg.heads, cfg.idx_heads
        off = 16 * layer
        s = cfg.seed
        self.q = torch.empty((n_rows, H, 512), dtype=torch.bfloat16, device=dev)
        csa2_synth_normal(s, synth.T_Q + off, 0, self.q)
        self.sink = None
        if cfg.extra.get("sink"):
            # per-head sink logits, N(0,1) rounded to bf16, kept in fp32
            self.sink = torch.empty((H,), dtype=torch.float32, device=dev)
            csa2_synth_normal(s, synth.T_SINK + off, 0, self.sink)
        if role not in ("reuse", "dense"):
            self.q_idx = torch.empty((n_rows, Hi, 128), dtype=torch.bfloat16, device=dev)
            csa2_synth_normal(s, synth.T_QIDX + off, 0, self.q_idx)
            self.w = torch.empty((n_rows, Hi), dtype=torch.float32, device=dev)
            csa2_synth_uniform(s, synth.T_W + off, 0, self.w)
        # sliding window: the row's own 128 8-bit entries
        n_swa = int(swa_first_tok[-1] + cfg.window) if n_rows else 0
        self.swa_codes, self.swa_scales = _planes(max(n_swa, 1), SWA_FP8, dev)
        _fill_packed(SWA_FP8, s, synth.T_SWA + off, 512, 0, n_swa, self.swa_codes, self.swa_scales, dev=dev)
        self.swa_first = torch.as_tensor(np.asarray(swa_first_tok, np.int64), device=dev)
        self.swa_count = torch.full((n_rows,), cfg.window, dtype=torch.int32, device=dev)
        if source is not None:
            # the positions (and counts) of the last Full or Reindex layer
            self.idx, self.idx_count = source.idx, source.idx_count
        elif role == "dense":
            self.idx = self.idx_count = None
        else:
            self.idx = torch.empty((n_rows, 512), dtype=torch.int32, device=dev)
            self.idx_count = torch.empty((n_rows,), dtype=torch.int32, device=dev)
        self.o_partial = torch.empty((n_rows, H, 512), dtype=torch.float32, device=dev)
        self.lse = torch.empty((n_rows, H), dtype=torch.float32, device=dev)
        self.out = torch.empty((n_rows, H, 512), dtype=torch.float32, device=dev)


class Workload:
    """All device buffers of one configuration; ``step()`` runs the hot path."""

    def __init__(self, cfg: Config, copies: int = 1, dev="cuda", separate: bool = False,
                 two_call_select: bool = False):
        self.cfg = cfg
        self.separate = separate
        self.two_call_select = two_call_select
        self.dev = dev
        L = cfg.lens
        base = cfg.req_base
        self.n_entries = int(L.sum())
        self.sigma = 512 ** -0.5
        # ---- rows
        if cfg.mode == "prefill":
            t = np.arange(cfg.prefill_tokens - cfg.prefill_rows, cfg.prefill_tokens, dtype=np.int64)
            n_vis = t // cfg.tokens_per_entry
            req = np.zeros(cfg.prefill_rows, np.int32)
            swa_first = t - (cfg.window - 1) - (t[0] - (cfg.window - 1))   # row i: tokens t-127 .. t
        else:
            n_vis = L.copy()
            req = np.arange(cfg.n_req, dtype=np.int32)
            swa_first = np.arange(cfg.n_req, dtype=np.int64) * cfg.window
        self.n_rows = len(req)
        self.n_vis_host = n_vis.astype(np.int64)
        self.max_vis = int(n_vis.max())
        self.req = torch.as_tensor(req, device=dev)
        self.n_vis = torch.as_tensor(n_vis.astype(np.int32), device=dev)
        self.rows = make_rows(self.req, self.n_vis, self.max_vis)
        # ---- global KV (MAIN + INDEX planes), logical entry = base[req] + pos
        if cfg.page_entries:
            P = cfg.page_entries
            pages_per_req = (L + P - 1) // P
            n_pages = int(pages_per_req.sum())
            perm = synth.page_permutation(cfg.seed, n_pages)
            max_pages = int(pages_per_req.max())
            table = np.zeros((cfg.n_req, max_pages), np.int32)
            k = 0
            for r in range(cfg.n_req):
                table[r, :pages_per_req[r]] = perm[k:k + pages_per_req[r]]
                k += pages_per_req[r]
            self.page_table_host = table
            self.page_table = torch.as_tensor(table, device=dev)
            n_slots = n_pages * P
        else:
            self.page_table_host = None
            self.page_table = None
            n_slots = self.n_entries
        self.n_slots = n_slots
        main0 = _planes(n_slots, MAIN_FP4, dev)
        idx0 = _planes(n_slots, INDEX_MXFP4, dev)
        self._fill_kv(main0, idx0)
        self.kv_copies = [(main0, idx0)]
        for _ in range(1, copies):
            self.kv_copies.append(((main0[0].clone(), main0[1].clone()), (idx0[0].clone(), idx0[1].clone())))
        stride = int(L.max()) if cfg.page_entries == 0 else 0
        self.kvs = [make_kv(m[0], m[1], i[0], i[1], n_slots, cfg.page_entries, self.page_table,
                            req_stride=stride if len(set(L.tolist())) == 1 else 0)
                    for (m, i) in self.kv_copies]
        if cfg.page_entries == 0 and len(set(L.tolist())) != 1:
            raise ValueError("contiguous layout needs equal contexts")
        # ---- layers
        self.layers = []
        source = None
        for li, role in enumerate(cfg.roles):
            if role == "reuse" and source is None:
                raise ValueError("a Reuse layer needs an earlier Full or Reindex layer")
            layer = Layer(cfg, self.n_rows, li, swa_first, dev, role=role,
                          source=source if role == "reuse" else None)
            if role != "reuse":
                source = layer
            self.layers.append(layer)
        if cfg.roles[0] not in ("full", "reindex", "prefill", "dense"):
            raise ValueError("the first layer of a step must select its own positions")
        self.graphs = None
        # ---- intermediates
        self.nv8 = (self.max_vis + 7) // 8 * 8
        mode = cfg.mode
        self.full = mode in ("full", "prefill", "mixed", "csa")
        if self.full:
            self.scores = torch.empty((self.n_rows, self.nv8), dtype=torch.float32, device=dev)
            self.block_max = _padded_rows(self.n_rows, self.nv8 // 8, dev)
        if mode in ("full", "mixed", "reindex"):
            self.pool = torch.empty((self.n_rows, 2048), dtype=torch.int32, device=dev)
            self.pool_count = torch.empty((self.n_rows,), dtype=torch.int32, device=dev)
            self.pool_scores = torch.empty((self.n_rows, 16384), dtype=torch.float32, device=dev)
        elif mode in ("prefill", "csa"):
            # the selection's 512-block pool (an intermediate of the step)
            self.pool = torch.empty((self.n_rows, 512), dtype=torch.int32, device=dev)
            self.pool_count = torch.empty((self.n_rows,), dtype=torch.int32, device=dev)
        ws = (csa2_dense_attn_workspace_size(self.n_rows, cfg.heads, self.max_vis) if mode == "dense"
              else csa2_attn_workspace_size(self.n_rows, cfg.heads))
        self.workspace = torch.empty(max(ws, 256) // 4, dtype=torch.float32, device=dev) if ws else None
        if mode == "reindex":
            pools = np.stack([synth.given_pool(cfg.seed, r, int(L[r]) // 8, 2048) for r in range(self.n_rows)])
            self.pool.copy_(torch.as_tensor(pools))
            self.pool_count.fill_(2048)
        torch.cuda.synchronize()

    def micro_batch(self) -> "Workload":
        """Another batch over the same cache and query-side inputs, with its
        own per-step buffers (scores, block maxima, pool, positions, outputs,
        workspace), so that its step can run on another stream while this
        one's runs."""
        import copy
        mb = copy.copy(self)
        for name in ("scores", "block_max", "pool", "pool_count", "pool_scores", "workspace"):
            t = getattr(self, name, None)
            if t is not None:
                setattr(mb, name, _padded_rows(t.shape[0], t.shape[1], self.dev) if name == "block_max" else t.clone())
        mb.layers = []
        new_sel = {}
        for layer in self.layers:
            nl = copy.copy(layer)
            if layer.role == "reuse":
                src = new_sel[id(layer.idx)]
                nl.idx, nl.idx_count = src.idx, src.idx_count
            elif layer.idx is not None:
                nl.idx, nl.idx_count = torch.empty_like(layer.idx), torch.empty_like(layer.idx_count)
                new_sel[id(layer.idx)] = nl
            nl.o_partial, nl.lse, nl.out = (torch.empty_like(layer.o_partial), torch.empty_like(layer.lse),
                                            torch.empty_like(layer.out))
            mb.layers.append(nl)
        mb.graphs = None
        torch.cuda.synchronize()
        return mb

    # --------------------------------------------------------------- setup
    def _fill_kv(self, main, idx):
        cfg = self.cfg
        L = cfg.lens
        base = cfg.req_base
        if cfg.page_entries == 0:
            _fill_packed(MAIN_FP4, cfg.seed, synth.T_LATENT, 512, 0, self.n_entries, main[0], main[1], dev=self.dev)
            _fill_packed(INDEX_MXFP4, cfg.seed, synth.T_IDXKEY, 128, 0, self.n_entries, idx[0], idx[1],
                         boost=cfg.boost, dev=self.dev)
            return
        P = cfg.page_entries
        for r in range(cfg.n_req):
            pos = np.arange(L[r], dtype=np.int64)
            slots = self.page_table_host[r, pos // P].astype(np.int64) * P + pos % P
            sl = torch.as_tensor(slots, device=self.dev)
            _fill_packed(MAIN_FP4, cfg.seed, synth.T_LATENT, 512, int(base[r]), int(L[r]), main[0], main[1],
                         slots=sl, dev=self.dev)
            _fill_packed(INDEX_MXFP4, cfg.seed, synth.T_IDXKEY, 128, int(base[r]), int(L[r]), idx[0], idx[1],
                         slots=sl, boost=cfg.boost, dev=self.dev)

    # --------------------------------------------------------------- the step
    @staticmethod
    def _mark(marks, name, which):
        if marks and name in marks:
            marks[name][which].record()

    def run_full(self, layer: "Layer", kv, stream=None, marks=None):
        m = self._mark
        m(marks, "index_score", 0)
        if self.cfg.mode == "prefill":
            # the chunk's rows are tokens of request 0: one scan of its keys serves them all
            csa2_index_score_shared(kv, self.rows, 0, layer.q_idx, layer.w, scores=self.scores,
                                    block_max=self.block_max, stream=stream)
        else:
            csa2_index_score(kv, self.rows, layer.q_idx, layer.w, scores=self.scores, block_max=self.block_max,
                             stream=stream)
        m(marks, "index_score", 1)
        if self.cfg.mode in ("prefill", "csa"):
            # top-512 over every visible score (no 2,048-block pool): a row's
            # top-512 positions lie in its 512 best blocks (a block ranked
            # above a top-512 position's block holds a distinct better position),
            # so the fused selection with a pool of 512 blocks returns exactly
            # the top-512 of all visible scores
            m(marks, "select", 0)
            csa2_select_full(self.block_max, self.scores, self.n_vis, self.max_vis, self.pool, self.pool_count,
                             layer.idx, layer.idx_count, n_pool_blocks=512, k=512, stream=stream)
            m(marks, "select", 1)
        elif self.two_call_select:
            m(marks, "select_blocks", 0)
            csa2_select_topk(self.block_max, 2048, self.pool, self.pool_count, n_cols=self.n_vis, cols_div=8,
                             max_cols=self.nv8 // 8, stream=stream)
            m(marks, "select_blocks", 1)
            m(marks, "select_positions", 0)
            csa2_select_topk(self.scores, 512, layer.idx, layer.idx_count, n_cols=self.pool_count, cols_mul=8,
                             pool_blocks=self.pool, keys_by_id=True, max_cols=16384, stream=stream)
            m(marks, "select_positions", 1)
        else:
            m(marks, "select", 0)
            csa2_select_full(self.block_max, self.scores, self.n_vis, self.max_vis, self.pool, self.pool_count,
                             layer.idx, layer.idx_count, stream=stream)
            m(marks, "select", 1)
        self._attend(layer, kv, stream, marks)

    def run_reindex(self, layer: "Layer", kv, stream=None, marks=None):
        m = self._mark
        m(marks, "index_score", 0)
        csa2_index_score(kv, self.rows, layer.q_idx, layer.w, scores=self.pool_scores,
                         pool_blocks=self.pool, pool_count=self.pool_count, stream=stream)
        m(marks, "index_score", 1)
        m(marks, "select_positions", 0)
        csa2_select_topk(self.pool_scores, 512, layer.idx, layer.idx_count, n_cols=self.pool_count, cols_mul=8,
                         pool_blocks=self.pool, keys_by_id=False, max_cols=16384, stream=stream)
        m(marks, "select_positions", 1)
        self._attend(layer, kv, stream, marks)

    def _attend(self, layer, kv, stream, marks=None):
        """Sparse + window attention in one pass (csa2_sparse_swa_attn); with
        separate=True the two-call form csa2_sparse_attn -> csa2_swa_merge."""
        m = self._mark
        if self.separate:
            m(marks, "sparse_attn", 0)
            csa2_sparse_attn(kv, self.rows, layer.q, layer.idx, layer.idx_count, self.sigma, layer.o_partial,
                             layer.lse, workspace=self.workspace, stream=stream)
            m(marks, "sparse_attn", 1)
            m(marks, "swa_merge", 0)
            csa2_swa_merge(layer.swa_codes, layer.swa_scales, layer.swa_first, layer.swa_count, layer.q,
                           self.sigma, layer.out, o_partial=layer.o_partial, lse=layer.lse, workspace=self.workspace,
                           stream=stream)
            m(marks, "swa_merge", 1)
        else:
            m(marks, "attention", 0)
            if layer.role == "dense":
                csa2_dense_swa_attn(kv, self.rows, layer.q, self.sigma, layer.out, swa_codes=layer.swa_codes,
                                    swa_scales=layer.swa_scales, swa_first=layer.swa_first,
                                    swa_count=layer.swa_count, sink=layer.sink, lse=layer.lse,
                                    workspace=self.workspace, stream=stream)
            else:
                csa2_sparse_swa_attn(kv, self.rows, layer.q, layer.idx, layer.idx_count, layer.swa_codes,
                                     layer.swa_scales, layer.swa_first, layer.swa_count, self.sigma, layer.out,
                                     sink=layer.sink, workspace=self.workspace, stream=stream)
            m(marks, "attention", 1)

    def step(self, copy: int = 0, stream=None, marks=None):
        """One pass of the hot path over every layer.  `marks` maps step names
        to (start, end) events recorded around that call (first layer only)."""
        kv = self.kvs[copy % len(self.kvs)]
        for i, layer in enumerate(self.layers):
            mk = marks if i == 0 else None
            if layer.role in ("full", "prefill"):
                self.run_full(layer, kv, stream, mk)
            elif layer.role == "reindex":
                self.run_reindex(layer, kv, stream, mk)
            else:
                self._attend(layer, kv, stream, mk)

    # --------------------------------------------------------------- graphs
    def capture_graphs(self):
        """Capture one whole step per KV copy as a HIP graph (torch's graph
        capture of the current stream; every call of the step is a kernel
        launch of libcsa2 on that stream, nothing else: no memset, no
        allocation).  Each copy's step runs eagerly once before capture."""
        for c in range(len(self.kvs)):
            self.step(copy=c)
        torch.cuda.synchronize()
        graphs = []
        for c in range(len(self.kvs)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step(copy=c)
            graphs.append(g)
        torch.cuda.synchronize()
        self.graphs = graphs

    def replay(self, copy: int = 0):
        """Replay the captured step of KV copy `copy` on the current stream."""
        self.graphs[copy % len(self.graphs)].replay()

    # --------------------------------------------------------------- bytes
    def algorithmic_bytes(self) -> dict:
        """Bytes the method must move per step: indexer keys scored, selected
        main entries gathered, window entries, queries in, outputs out.  Data
        that several rows share is counted once: the rows of a chunked
        prefill read one request's keys (its largest visible prefix) and
        overlapping windows (rows + window - 1 entries).  A Reuse layer moves
        its gathered entries, window, query and output, no indexer bytes."""
        cfg = self.cfg
        H = cfg.heads
        rows = self.n_rows
        prefill = cfg.mode == "prefill"
        roles = [layer.role for layer in self.layers]
        n_layers = len(roles)
        n_index = sum(r not in ("reuse", "dense") for r in roles)
        d = {}
        n_full = sum(r in ("full", "prefill") for r in roles)
        if n_full:
            keys = int(self.n_vis_host.max()) if prefill else int(self.n_vis_host.sum())
            d["index_keys_full"] = n_full * keys * 68
        n_reindex = sum(r == "reindex" for r in roles)
        if n_reindex:
            pool_pos = int(np.minimum(self.n_vis_host, 16384).sum()) if cfg.mode != "reindex" else rows * 16384
            d["index_keys_pool"] = n_reindex * pool_pos * 68
        if cfg.mode == "dense":
            d["dense_main"] = n_layers * int(self.n_vis_host.sum()) * 288
        else:
            sel = int(np.minimum(self.n_vis_host, 512).sum())
            d["gathered_main"] = n_layers * sel * 288
        d["swa"] = n_layers * (rows + cfg.window - 1 if prefill else rows * cfg.window) * 544
        d["q"] = n_layers * rows * H * 512 * 2 + n_index * rows * (cfg.idx_heads * 128 * 2 + cfg.idx_heads * 4)
        d["out"] = n_layers * rows * H * 512 * 4
        d["total"] = sum(d.values())
        return d
