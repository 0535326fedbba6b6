/*
 * csa2.h -- C-ABI of the CSA2 decode hot path on AMD Instinct MI355X (gfx950).
 *
 * CSA2 is the compressed sparse attention of a DeepSeek-V4.1-Flash-style
 * layer.  For every query row it
 *   1. scores each visible cached position with the lightning indexer,
 *      I_s = sum_h w_h * ReLU(q_h . K_s), over 128-channel MXFP4 keys
 *      ['DeepSeek-V4' paper page, section 2.3.1, index-score equation;
 *       section 2.3.4: indexer attention in FP4];
 *   2. keeps the 2,048 best aligned 8-position blocks (ranked by their maximum
 *      score) as a 16,384-position candidate pool, or re-scores a given pool
 *      in a Reindex layer, and takes the top 512 positions
 *      ['DeepSeek V4.1 Flash architecture analysis' page, hierarchical sparse
 *       indexer section; 'DeepSeek-V4' page, section 2.3.1, top-k selector];
 *   3. gathers those positions' 512-channel FP4 latent entries, dequantises
 *      them and attends with the latent as key and value (shared-KV MQA,
 *      absorbed-MLA style), jointly with a 128-token 8-bit sliding-window
 *      branch and an optional sink ['DeepSeek-V4' page, sections 2.3.1
 *      "Shared Key-Value MQA" and 2.3.3; MLA article, section 4].
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller; descriptor
 *     structs (csa2_kv, csa2_rows) are HOST memory read during the call.  The
 *     library keeps no pointer after a call returns and allocates nothing.
 *   - `stream` is a hipStream_t (NULL: the null stream).  Work is enqueued
 *     and the call returns without synchronising.
 *   - Arguments are validated on the host before any launch; on error the
 *     call returns a non-zero csa2_status, enqueues nothing and leaves the
 *     outputs untouched; csa2_last_error() gives a message (per thread).
 *     Faults during execution surface at the caller's next synchronisation.
 *   - Data preconditions that are not checked: inputs are finite; pool
 *     blocks of a row are distinct, ascending and visible; idx entries are
 *     below the row's visible count; slot ids are distinct and in range.
 *   - All outputs are bitwise reproducible run to run.
 *
 * Storage formats (one "entry" = one compressed KV position)
 *   MAIN  (latent KV, 512 ch): codes [256 B] = E2M1 pairs, channel 2j in the
 *         low nibble of byte j; scales [32 B] = one E4M3 per 16 channels,
 *         s = E4M3(fl32(amax/6)) rounded to nearest even, saturating at 448;
 *         code = E2M1(fl32(x/s)) nearest even, saturating at 6.  288 B.
 *   INDEX (indexer keys / queries, 128 ch): codes [64 B] E2M1 as above;
 *         scales [4 B] E8M0 per 32 channels, e = floor(log2 amax) - 2
 *         clamped to [-127, 127], code = E2M1(x * 2^-e).  68 B.
 *   SWA   (sliding-window KV, 512 ch): codes [512 B] E4M3; scales [32 B]
 *         E8M0 per 16 channels, e = floor(log2 amax) - 8, code =
 *         E4M3(x * 2^-e) nearest even, saturating.  544 B.
 * Each kind is stored as two planes (codes, scales) indexed by entry id.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_ABI_VERSION 5

/* The enums are int-sized in C; in C++ they are given int as their fixed
 * underlying type, so that every int a C caller passes (an invalid one is
 * rejected with a status) is a valid value of the parameter's type. */
#ifdef __cplusplus
#define CSA2_INT_ENUM : int
#else
#define CSA2_INT_ENUM
#endif

typedef enum CSA2_INT_ENUM {
    CSA2_OK = 0,
    CSA2_ERR_NULL = 1,        /* a required pointer is NULL */
    CSA2_ERR_SHAPE = 2,       /* inconsistent sizes or strides */
    CSA2_ERR_RANGE = 3,       /* a size or count outside its allowed range */
    CSA2_ERR_ALIGN = 4,       /* a pointer or stride is not aligned as required */
    CSA2_ERR_UNSUPPORTED = 5, /* a head count or dtype the library does not handle */
    CSA2_ERR_WORKSPACE = 6,   /* reserved: no entry point of this version returns it */
    CSA2_ERR_HIP = 7          /* the HIP runtime reported an error at launch */
} csa2_status;

typedef enum CSA2_INT_ENUM { CSA2_BF16 = 0, CSA2_F32 = 1 } csa2_dtype;
typedef enum CSA2_INT_ENUM { CSA2_MAIN_FP4 = 0, CSA2_INDEX_MXFP4 = 1, CSA2_SWA_FP8 = 2 } csa2_kind;

/* Fixed constants of the method: 'candidate_topk_blocks' 2,048,
 * 'candidate_block_size' 8, 'index_topk' 512, sliding window 128. */
#define CSA2_LATENT 512
#define CSA2_INDEX_DIM 128
#define CSA2_POOL_BLOCKS 2048
#define CSA2_BLOCK 8
#define CSA2_TOPK 512
#define CSA2_WINDOW 128
#define CSA2_MAX_SELECT 2048  /* largest k csa2_select_topk accepts */
#define CSA2_MAX_POOL_BLOCKS 2048  /* largest pool csa2_select_full builds */

/* The global (compressed) KV cache: MAIN and INDEX planes indexed by entry id.
 *   page_entries == 0: contiguous; entry(req, pos) = req * req_stride + pos.
 *   page_entries  > 0: paged; entry(req, pos) =
 *        page_table[req * max_pages + pos / page_entries] * page_entries
 *        + pos % page_entries; page_entries must be a multiple of 16.
 * Every plane pointer must be 256-byte aligned. */
typedef struct csa2_kv {
    const uint8_t* main_codes;   /* [n_slots][256] (may be NULL for scoring-only calls) */
    const uint8_t* main_scales;  /* [n_slots][32]  */
    const uint8_t* idx_codes;    /* [n_slots][64]  (may be NULL for attention-only calls) */
    const uint8_t* idx_scales;   /* [n_slots][4]   */
    int64_t n_slots;             /* entries held by each plane */
    int32_t page_entries;        /* 0 = contiguous */
    int32_t max_pages;           /* row length of page_table */
    const int32_t* page_table;   /* device [n_req][max_pages], paged layout only */
    int64_t req_stride;          /* contiguous layout only */
} csa2_kv;

/* Query rows.  For decode a row is a request; for chunked prefill a row is a
 * query token of a request, with its own visible count. */
typedef struct csa2_rows {
    const int32_t* req;    /* device [n_rows]: request id of each row */
    const int32_t* n_vis;  /* device [n_rows]: visible entries, positions [0, n_vis) */
    int32_t n_rows;
    int32_t max_vis;       /* host: an upper bound on every n_vis (sizes the grid) */
} csa2_rows;

int csa2_abi_version(void);
/* Text of a status code; any int is accepted (codes outside csa2_status give
 * "unknown status"). */
const char* csa2_status_str(int status);
const char* csa2_last_error(void);

/* ---------------------------------------------------------------- packing
 * Quantise n rows of `src` (bf16 or fp32; row r at src + r * src_row_stride
 * elements; 512 channels for MAIN/SWA, 128 for INDEX) and write the codes and
 * scales of row r to entry slots[r] (slots NULL: entry r).  The write path of
 * the cache ('890 bytes/token' section of the V4.1-Flash architecture page;
 * quantisation after RoPE, 'KV cache diet' page).  Not part of the decode step. */
csa2_status csa2_pack_kv(csa2_kind kind, const void* src, csa2_dtype src_dtype, int64_t n,
                         int64_t src_row_stride, uint8_t* codes, uint8_t* scales,
                         const int64_t* slots, void* stream);

/* ---------------------------------------------------------------- write path
 * Compressed cache entries built from projected token streams, normalised,
 * rotated and packed in one pass ('DeepSeek-V4' page, section 2.3.1,
 * compressed key-value entries; 2.3.2 for the non-overlapping form; 2.3.3
 * RMSNorm and partial RoPE; 'KV cache diet' page: quantisation after RoPE).
 * The streams are the layer's projections of its hidden states (C = H W^KV,
 * Z = H W^Z), computed by the caller: fp32, token rows of `row_stride`
 * elements, `width` channels (512 for MAIN, 128 for INDEX).
 *   Overlapping (cb, zb, bb given): entry i, per channel, is the softmax over
 *   the 2m logits za[m i + k] + ba[k] and zb[m (i-1) + k] + bb[k] (k < m)
 *   weighting ca[m i + k] and cb[m (i-1) + k]; entry 0 has no b part.
 *   Non-overlapping (cb, zb, bb NULL): the softmax over za[m i + k] + ba[k]
 *   weighting ca[m i + k].
 * Then, if norm_weight [width] is given, y = x / sqrt(mean(x^2) + eps) *
 * norm_weight; if rope, channel pairs (width - 64 + 2j, width - 63 + 2j)
 * rotate by (pos0 + m i) * 10000^(-2j/64).  Entry i (i < n_tok / m) is
 * written packed (kind MAIN_FP4 or INDEX_MXFP4, the csa2_pack_kv rules) to
 * slots[i] (NULL: slot i); `values` [n_tok/m][width] (may be NULL) receives
 * the fp32 values that were packed.  1 <= m <= 1,024. */
typedef struct csa2_compress_streams {
    const float* ca;
    const float* za;
    const float* cb;          /* NULL: non-overlapping compression */
    const float* zb;
    const float* ba;          /* [m][width] */
    const float* bb;          /* [m][width], overlapping only */
    int64_t n_tok;
    int64_t row_stride;       /* elements between token rows (>= width, multiple of 4) */
    int32_t m;
} csa2_compress_streams;
csa2_status csa2_compress_pack(csa2_kind kind, const csa2_compress_streams* streams,
                               const float* norm_weight, float eps, int32_t rope, int64_t pos0,
                               float* values, uint8_t* codes, uint8_t* scales, const int64_t* slots,
                               void* stream);

/* ---------------------------------------------------------------- indexer
 * Lightning-indexer scores ('DeepSeek-V4' page, section 2.3.1):
 *   q_idx [n_rows][n_idx_heads][128] (bf16 or fp32) is quantised to MXFP4 per
 *   (row, head, 32 channels) with the INDEX rule; w [n_rows][n_idx_heads] fp32.
 *   d_h = q_h . K_s, exact, rounded once to fp32 (nearest even);
 *   score_s = fma-fold over h = 0 .. n_idx_heads-1 of (w_h, max(d_h, +0)),
 *   starting from +0; -0 is returned as +0.
 * Full scan (pool_blocks == NULL): every position s < n_vis[row].
 *   scores [n_rows][scores_stride]: columns [0, n_vis) hold scores, columns
 *   [n_vis, roundup(n_vis, 8)) hold -inf; scores_stride >= roundup(max_vis, 8).
 *   block_max [n_rows][block_max_stride]: column j < ceil(n_vis/8) holds the
 *   max over positions [8j, min(8j+8, n_vis)).  Either output may be NULL.
 * Pool mode (Reindex; pool_blocks != NULL): only the blocks
 *   pool_blocks[row * pool_stride + j], j < pool_count[row] (<= 2,048), are
 *   scored; column 8j+i of `scores` holds the score of position
 *   8*pool_blocks[..j] + i, or -inf if that position is >= n_vis.
 *   block_max must be NULL.
 * n_idx_heads in 1..64.  Requires kv->idx_codes / idx_scales. */
csa2_status csa2_index_score(const csa2_kv* kv, const csa2_rows* rows,
                             const void* q_idx, csa2_dtype q_dtype, int32_t n_idx_heads,
                             const float* w,
                             const int32_t* pool_blocks, int64_t pool_stride,
                             const int32_t* pool_count,
                             float* scores, int64_t scores_stride,
                             float* block_max, int64_t block_max_stride,
                             void* stream);

/* Chunked prefill: the same full scan for query rows that all belong to ONE
 * request `req` (host value; rows->req is not read and may be NULL), each row
 * with its own visible count rows->n_vis[row] (in a causal chunk the later
 * tokens see more entries).  The rows share the key stream: a workgroup loads
 * each 16-key tile once and scores it against up to 16 rows, so the scan is
 * bound by the MFMA and the score writes instead of by re-reading the keys
 * once per row ('DeepSeek-V4' page, section 2.3.1: the indexer scores every
 * query token against every preceding compressed entry).  The outputs, their
 * layout and their bits are those of csa2_index_score's full scan.
 * 0 <= req < number of requests the cache holds; n_idx_heads in 1..16. */
csa2_status csa2_index_score_shared(const csa2_kv* kv, const csa2_rows* rows, int32_t req,
                                    const void* q_idx, csa2_dtype q_dtype, int32_t n_idx_heads,
                                    const float* w,
                                    float* scores, int64_t scores_stride,
                                    float* block_max, int64_t block_max_stride,
                                    void* stream);

/* ---------------------------------------------------------------- top-k
 * Exact row-wise top-k ('DeepSeek-V4' page, section 2.3.1, top-k selector;
 * V4.1-Flash architecture page, hierarchical sparse indexer: blocks ranked by
 * their maximum, ties to the lower position).
 * Row r has c_r = ceil(n_cols[r] * cols_mul / cols_div) candidate columns
 * (n_cols NULL: max_cols), c_r <= max_cols.  Column c has id
 *   id(c) = c                                          (ids and pool_blocks NULL)
 *   id(c) = ids[r * ids_stride + c]                    (ids given)
 *   id(c) = 8 * pool_blocks[r * pool_stride + c/8] + c%8   (pool_blocks given)
 * and key keys[r * key_stride + (keys_by_id ? id(c) : c)].  Keys equal to
 * -inf are absent.  The min(k, present) columns first in (key descending,
 * id ascending) are selected.  Column order must be id order: a row's ids
 * strictly ascending over its c_r columns, its pool blocks ascending (not
 * checked).  The selected ids are written ascending to
 * out_ids[r * out_stride ..], the rest of the k slots get -1, and
 * out_count[r] the number selected.
 * 1 <= k <= 2,048; max_cols <= 2^24; cols_mul, cols_div in 1..8; ids and
 * pool_blocks are exclusive; keys_by_id needs pool_blocks; ids_stride >=
 * max_cols.
 * workspace: device scratch of csa2_select_topk_workspace(n_rows, max_cols, k)
 * bytes, 256-B aligned.  This version keeps its whole selection in LDS and
 * registers, so the size is 0 for every shape and the workspace may be NULL;
 * a non-zero size passed with a NULL pointer is an error. */
size_t csa2_select_topk_workspace(int32_t n_rows, int32_t max_cols, int32_t k);
csa2_status csa2_select_topk(const float* keys, int64_t key_stride,
                             const int32_t* ids, int64_t ids_stride,
                             const int32_t* n_cols, int32_t cols_mul, int32_t cols_div,
                             const int32_t* pool_blocks, int64_t pool_stride, int32_t keys_by_id,
                             int32_t n_rows, int32_t max_cols, int32_t k,
                             int32_t* out_ids, int64_t out_stride, int32_t* out_count,
                             void* workspace, size_t workspace_bytes, void* stream);

/* The Full layer's selection in one pass per row (V4.1-Flash architecture
 * page, hierarchical sparse indexer: the first Full layer keeps up to 2,048
 * groups of 8 positions ranked by their maximum and picks its own top-512
 * among them).  Same result as two csa2_select_topk calls:
 *   pool = top-n_pool_blocks of block_max[r][0 .. ceil(n_vis[r]/8)) by
 *          (maximum descending, block ascending), ids ascending, -1 padded,
 *          count in pool_count[r];
 *   idx  = top-k of scores[r][p] over the pool's positions p = 8 b + i
 *          (i < 8), ids ascending, -1 padded, count in idx_count[r].
 * block_max and scores are csa2_index_score's full-scan outputs (scores
 * beyond n_vis up to a multiple of 8 hold -inf); scores rows 16-B aligned
 * (scores_stride a multiple of 4).  1 <= n_pool_blocks <= 2,048,
 * 1 <= k <= 2,048. */
csa2_status csa2_select_full(const float* block_max, int64_t block_max_stride,
                             const float* scores, int64_t scores_stride,
                             const int32_t* n_vis, int32_t n_rows, int32_t max_vis,
                             int32_t n_pool_blocks, int32_t k,
                             int32_t* pool, int64_t pool_stride, int32_t* pool_count,
                             int32_t* idx, int64_t idx_stride, int32_t* idx_count,
                             void* stream);

/* ---------------------------------------------------------------- attention
 * Core attention of CSA2 ('DeepSeek-V4' page, section 2.3.1 "Shared Key-Value
 * MQA": each selected compressed entry is both key and value; section 2.3.3:
 * the sliding-window entries join the selected ones in the same softmax, and
 * a per-head sink logit adds exp(sink_h) to its denominator; MLA article,
 * section 4: the query is the absorbed query in the 512-channel latent space).
 * For a row and head h, with z_j = softmax_scale * q_h . E_j over the row's
 * entries E_j (dequantised, exact):
 *   o[row][h][:] = sum_j e^(z_j) E_j / (sum_j e^(z_j) [+ e^(sink_h)]),
 *   lse[row][h]  = ln(sum_j e^(z_j) [+ e^(sink_h)]), -inf (o = 0) if empty.
 * Entry sets: the SELECTED entries are the MAIN entries of positions
 * idx[row * idx_stride + j], j < idx_count[row] (<= 512, positions < n_vis);
 * the WINDOW entries are SWA entries swa_first[row] .. + swa_count[row] - 1
 * (<= 128) of the planes swa_codes [swa_slots][512] / swa_scales [.][32].
 * q [n_rows][n_heads][512] bf16 (fp32 is rounded to bf16 on the way in);
 * n_heads 16, 32, 48, 64 or 128; outputs fp32.  q, o/out 16-B aligned.
 * workspace: NULL, or csa2_attn_workspace_size(n_rows, n_heads) bytes,
 * 256-B aligned, no initialisation, not kept between calls.  With it, a call
 * with few rows spreads each row's entry list over several workgroups and
 * joins their partial results in a second pass; without it (or when the size
 * is 0) every row and group of 16 heads is one workgroup.  Either way a row's
 * outputs are the same bits, whatever the other rows of the call: its entry
 * list (selected entries padded to a multiple of 64, then the window) is cut
 * into units of 192 entries whose softmax max and sum start afresh, and the
 * units are joined left to right by one fixed sequence of operations
 * (bitwise batch invariance, 'DeepSeek-V4' page, section 3.3). */
size_t csa2_attn_workspace_size(int32_t n_rows, int32_t n_heads);

/* Selected entries only: o_partial / lse of the sparse branch. */
csa2_status csa2_sparse_attn(const csa2_kv* kv, const csa2_rows* rows,
                             const void* q, csa2_dtype q_dtype, int32_t n_heads,
                             const int32_t* idx, int64_t idx_stride, const int32_t* idx_count,
                             float softmax_scale, float* o_partial, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Window branch merged with a sparse-branch result through its log-sum-exp:
 * out = joint softmax over {the entries behind (o_partial, lse)} + {window}
 * (+ sink).  o_partial / lse NULL: window only.  sink [n_heads] or NULL.
 * out may alias o_partial. */
csa2_status csa2_swa_merge(const uint8_t* swa_codes, const uint8_t* swa_scales, int64_t swa_slots,
                           const int64_t* swa_first, const int32_t* swa_count, int32_t n_rows,
                           const void* q, csa2_dtype q_dtype, int32_t n_heads, float softmax_scale,
                           const float* sink, const float* o_partial, const float* lse,
                           float* out, void* workspace, size_t workspace_bytes, void* stream);

/* Both branches in one pass (the decode step's form): out = joint softmax
 * over selected + window entries (+ sink); lse (may be NULL) of that joint
 * denominator. */
csa2_status csa2_sparse_swa_attn(const csa2_kv* kv, const csa2_rows* rows,
                                 const void* q, csa2_dtype q_dtype, int32_t n_heads,
                                 const int32_t* idx, int64_t idx_stride, const int32_t* idx_count,
                                 const uint8_t* swa_codes, const uint8_t* swa_scales, int64_t swa_slots,
                                 const int64_t* swa_first, const int32_t* swa_count, const float* sink,
                                 float softmax_scale, float* out, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Dense form for the heavily compressed branch ('DeepSeek-V4' page, section
 * 2.3.2: every m' = 128 tokens are compressed into one entry and the query
 * attends to ALL of them, no sparse selection; the same shared-KV MQA, and,
 * as section 2.3.3 adds, the same sliding-window branch and sink): the
 * entries of row r are the MAIN entries of its positions 0 .. n_vis[r]-1
 * (every visible compressed entry; rows->max_vis bounds them, at most
 * CSA2_MAX_DENSE), joined in one softmax with the window entries (swa_codes
 * NULL: no window) and the sink.  Same output conventions, numerics and
 * bitwise batch invariance as csa2_sparse_swa_attn (the entry list is the
 * row's entries padded to a multiple of 64, then the window, cut into units
 * of 768 entries folded left to right).  workspace: NULL or
 * csa2_dense_attn_workspace_size(n_rows, n_heads, rows->max_vis) bytes,
 * 256-B aligned, not kept between calls; with it a launch with few rows
 * spreads each row's units over several workgroups. */
#define CSA2_MAX_DENSE (1 << 22)
size_t csa2_dense_attn_workspace_size(int32_t n_rows, int32_t n_heads, int32_t max_vis);
csa2_status csa2_dense_swa_attn(const csa2_kv* kv, const csa2_rows* rows,
                                const void* q, csa2_dtype q_dtype, int32_t n_heads,
                                const uint8_t* swa_codes, const uint8_t* swa_scales, int64_t swa_slots,
                                const int64_t* swa_first, const int32_t* swa_count, const float* sink,
                                float softmax_scale, float* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * call as csa2_sparse_swa_attn without a workspace argument.  Where the call
 * would spread rows over several workgroups, its partial results go to a
 * device array the library owns instead: CSA2_ATTN_SCRATCH_BYTES per GPU,
 * held from the library's load on that GPU until the process ends, its
 * address looked up on the first call on each device.  The call itself
 * allocates and frees nothing.  Outputs are the bits csa2_sparse_swa_attn
 * gives with a workspace (and without one).  The scratch needs no clearing
 * (every partial a call folds is written earlier in that call), but it is
 * one array per GPU: calls that overlap on the same GPU (other streams, other
 * host threads) race on it and must be serialised by the caller.  A call
 * whose split pass would need more than CSA2_ATTN_SCRATCH_BYTES returns
 * CSA2_ERR_RANGE before any launch (no supported shape does: the split pass
 * is used up to 2,048 (row, head) pairs). */
#define CSA2_ATTN_SCRATCH_BYTES ((size_t)2048 * 4 * 514 * 4)
csa2_status csa2_sparse_swa_attn_noalloc(const csa2_kv* kv, const csa2_rows* rows,
                                         const void* q, csa2_dtype q_dtype, int32_t n_heads,
                                         const int32_t* idx, int64_t idx_stride, const int32_t* idx_count,
                                         const uint8_t* swa_codes, const uint8_t* swa_scales, int64_t swa_slots,
                                         const int64_t* swa_first, const int32_t* swa_count, const float* sink,
                                         float softmax_scale, float* out, float* lse, void* stream);

/* ---------------------------------------------------------------- streaming-read reference
 * Not a step of the method: the plain streaming read that the indexer scan's
 * HBM rate is measured against.  Reads the n_bytes of buf once (16-B
 * non-temporal loads, as the scan reads its keys, by 1,024 workgroups
 * striding over the buffer); out[g], g < CSA2_STREAM_XOR_WORDS, receives the
 * XOR of the 32-bit words workgroup g read (0 if none), so the XOR of all
 * out words is the XOR of the buffer's words.  buf 16-B aligned, n_bytes a
 * multiple of 16 (0: nothing to do, out untouched), out 4-B aligned with
 * room for CSA2_STREAM_XOR_WORDS words; device memory owned by the caller. */
#define CSA2_STREAM_XOR_WORDS 1024
csa2_status csa2_stream_xor(const void* buf, int64_t n_bytes, uint32_t* out, void* stream);

/* ---------------------------------------------------------------- synthetic inputs
 * Counter-based generator for seeded synthetic inputs (SplitMix64; Steele,
 * Lea & Flood 2014): base = mix64(seed * 0x9E3779B97F4A7C15 + tensor_id),
 * word(i) = mix64(base + (i+1) * 0x9E3779B97F4A7C15).
 * normal: element i = bf16 (nearest even) of (sum of the twelve 16-bit
 *   fields of words 3i..3i+2 - 393210) * 2^-16 (Irwin-Hall N(0,1)), for
 *   elements first .. first+n-1, written as bf16 or as the same value in fp32.
 * uniform: element i = (word(i) >> 40) * 2^-24, fp32. */
csa2_status csa2_synth_normal(uint64_t seed, uint32_t tensor_id, int64_t first, int64_t n,
                              csa2_dtype out_dtype, void* out, void* stream);
csa2_status csa2_synth_uniform(uint64_t seed, uint32_t tensor_id, int64_t first, int64_t n,
                               float* out, void* stream);
/* Multiply rows [0, n_rows) of x [n_rows][width] fp32 by 3 where the row's
 * position first_pos + r is boosted: word(pos) of stream (seed, boost_tensor)
 * below 0.05 * 2^64 (about 5% of positions). */
csa2_status csa2_synth_boost(uint64_t seed, uint32_t boost_tensor, int64_t first_pos, int64_t n_rows,
                             int32_t width, float* x, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
