// api.cpp -- the C-ABI of libcsa2: host-side argument validation, then the
// kernel launches.  No allocation, no synchronisation, no global device state
// besides the one-time LDS attribute of the attention kernels.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/csa2.h"
#include "csa2_device.h"
#include "csa2_launch.h"

namespace {

thread_local char g_err[512] = "";

csa2_status fail(csa2_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

csa2_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return CSA2_OK;
    return fail(CSA2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int log2_exact(int v) {
    if (v <= 0 || (v & (v - 1))) return -1;
    int s = 0;
    while ((1 << s) < v) ++s;
    return s;
}

csa2_status make_view(const csa2_kv* kv, bool need_main, bool need_idx, csa2::KvView* out) {
    if (!kv) return fail(CSA2_ERR_NULL, "kv descriptor is NULL");
    if (need_main && (!kv->main_codes || !kv->main_scales)) return fail(CSA2_ERR_NULL, "main KV planes are NULL");
    if (need_idx && (!kv->idx_codes || !kv->idx_scales)) return fail(CSA2_ERR_NULL, "indexer key planes are NULL");
    const void* planes[4] = {kv->main_codes, kv->main_scales, kv->idx_codes, kv->idx_scales};
    for (const void* p : planes)
        if (p && !aligned(p, 256)) return fail(CSA2_ERR_ALIGN, "KV plane pointers must be 256-byte aligned");
    if (kv->n_slots <= 0) return fail(CSA2_ERR_RANGE, "kv->n_slots must be positive");
    int shift = -1;
    if (kv->page_entries != 0) {
        shift = log2_exact(kv->page_entries);
        if (shift < 4) return fail(CSA2_ERR_RANGE, "page_entries must be a power of two >= 16 (got %d)", kv->page_entries);
        if (!kv->page_table) return fail(CSA2_ERR_NULL, "paged layout without a page table");
        if (kv->max_pages <= 0) return fail(CSA2_ERR_RANGE, "max_pages must be positive");
    } else if (kv->req_stride < 0) {
        return fail(CSA2_ERR_RANGE, "req_stride must be non-negative");
    }
    out->main_codes = kv->main_codes;
    out->main_scales = kv->main_scales;
    out->idx_codes = kv->idx_codes;
    out->idx_scales = kv->idx_scales;
    out->page_table = kv->page_table;
    out->req_stride = kv->req_stride;
    out->page_shift = shift;
    out->max_pages = kv->max_pages;
    return CSA2_OK;
}

csa2_status check_rows(const csa2_rows* rows) {
    if (!rows) return fail(CSA2_ERR_NULL, "rows descriptor is NULL");
    if (rows->n_rows < 0) return fail(CSA2_ERR_RANGE, "n_rows must be >= 0");
    if (rows->n_rows > 0 && (!rows->req || !rows->n_vis)) return fail(CSA2_ERR_NULL, "rows->req / rows->n_vis are NULL");
    if (rows->n_rows > 65535) return fail(CSA2_ERR_RANGE, "n_rows above 65535");
    if (rows->max_vis < 0 || rows->max_vis > (1 << 30)) return fail(CSA2_ERR_RANGE, "max_vis out of range");
    return CSA2_OK;
}

}  // namespace

extern "C" {

int csa2_abi_version(void) { return CSA2_ABI_VERSION; }

const char* csa2_status_str(int status) {
    switch (status) {
        case CSA2_OK: return "ok";
        case CSA2_ERR_NULL: return "null pointer";
        case CSA2_ERR_SHAPE: return "inconsistent shape";
        case CSA2_ERR_RANGE: return "value out of range";
        case CSA2_ERR_ALIGN: return "misaligned pointer or stride";
        case CSA2_ERR_UNSUPPORTED: return "unsupported configuration";
        case CSA2_ERR_WORKSPACE: return "workspace missing or too small";
        case CSA2_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* csa2_last_error(void) { return g_err; }

csa2_status csa2_pack_kv(csa2_kind kind, const void* src, csa2_dtype src_dtype, int64_t n,
                         int64_t src_row_stride, uint8_t* codes, uint8_t* scales,
                         const int64_t* slots, void* stream) {
    if (kind != CSA2_MAIN_FP4 && kind != CSA2_INDEX_MXFP4 && kind != CSA2_SWA_FP8)
        return fail(CSA2_ERR_UNSUPPORTED, "unknown kind %d", (int)kind);
    if (src_dtype != CSA2_BF16 && src_dtype != CSA2_F32) return fail(CSA2_ERR_UNSUPPORTED, "unknown dtype");
    if (n < 0) return fail(CSA2_ERR_RANGE, "n must be >= 0");
    if (n == 0) return CSA2_OK;
    if (!src || !codes || !scales) return fail(CSA2_ERR_NULL, "src / codes / scales is NULL");
    const int64_t width = kind == CSA2_INDEX_MXFP4 ? 128 : 512;
    if (src_row_stride < width) return fail(CSA2_ERR_SHAPE, "src_row_stride %lld < %lld channels", (long long)src_row_stride, (long long)width);
    const int64_t esz = src_dtype == CSA2_BF16 ? 2 : 4;
    if (!aligned(src, 16) || (src_row_stride * esz) % 16) return fail(CSA2_ERR_ALIGN, "src and its row stride must be 16-byte aligned");
    if (!aligned(codes, 256) || !aligned(scales, 256)) return fail(CSA2_ERR_ALIGN, "code and scale planes must be 256-byte aligned");
    if (n > ((int64_t)1 << 40)) return fail(CSA2_ERR_RANGE, "n too large");
    return hip_status(csa2::launch_pack((int)kind, src, src_dtype == CSA2_BF16, n, src_row_stride, codes, scales,
                                        slots, (hipStream_t)stream), "csa2_pack_kv launch");
}

csa2_status csa2_compress_pack(csa2_kind kind, const csa2_compress_streams* st, const float* norm_weight, float eps,
                               int32_t rope, int64_t pos0, float* values, uint8_t* codes, uint8_t* scales,
                               const int64_t* slots, void* stream) {
    if (kind != CSA2_MAIN_FP4 && kind != CSA2_INDEX_MXFP4)
        return fail(CSA2_ERR_UNSUPPORTED, "csa2_compress_pack packs MAIN or INDEX entries (kind %d)", (int)kind);
    if (!st) return fail(CSA2_ERR_NULL, "streams descriptor is NULL");
    if (st->m < 1 || st->m > 1024) return fail(CSA2_ERR_RANGE, "m must be in 1..1024 (got %d)", st->m);
    if (st->n_tok < 0 || st->n_tok > ((int64_t)1 << 40)) return fail(CSA2_ERR_RANGE, "n_tok out of range");
    const int width = kind == CSA2_MAIN_FP4 ? 512 : 128;
    const int64_t n_ent = st->n_tok / st->m;
    if (n_ent == 0) return CSA2_OK;
    if (!st->ca || !st->za || !st->ba || !codes || !scales) return fail(CSA2_ERR_NULL, "ca / za / ba / codes / scales is NULL");
    const bool overlap = st->cb || st->zb || st->bb;
    if (overlap && (!st->cb || !st->zb || !st->bb)) return fail(CSA2_ERR_NULL, "cb, zb and bb go together");
    if (st->row_stride < width || st->row_stride % 4) return fail(CSA2_ERR_SHAPE, "row_stride must be >= %d and a multiple of 4", width);
    const void* ptrs[6] = {st->ca, st->za, st->cb, st->zb, st->ba, st->bb};
    for (const void* p : ptrs)
        if (p && !aligned(p, 16)) return fail(CSA2_ERR_ALIGN, "stream and bias pointers must be 16-byte aligned");
    if ((norm_weight && !aligned(norm_weight, 16)) || (values && !aligned(values, 16)))
        return fail(CSA2_ERR_ALIGN, "norm_weight and values must be 16-byte aligned");
    if (!aligned(codes, 256) || !aligned(scales, 256)) return fail(CSA2_ERR_ALIGN, "code and scale planes must be 256-byte aligned");
    if (!(eps >= 0.0f) || eps > 1.0f) return fail(CSA2_ERR_RANGE, "eps must be in [0, 1]");
    if (pos0 < 0) return fail(CSA2_ERR_RANGE, "pos0 must be >= 0");
    csa2::CompressArgs a;
    a.m = st->m;
    a.ca = st->ca;
    a.za = st->za;
    a.cb = overlap ? st->cb : nullptr;
    a.zb = overlap ? st->zb : nullptr;
    a.ba = st->ba;
    a.bb = overlap ? st->bb : nullptr;
    a.stride = st->row_stride;
    a.n_ent = n_ent;
    a.norm_weight = norm_weight;
    a.eps = eps;
    a.rope = rope != 0;
    a.pos0 = pos0;
    return hip_status(csa2::launch_compress_pack(a, width, values, codes, scales, slots, (hipStream_t)stream),
                      "csa2_compress_pack launch");
}

csa2_status csa2_index_score(const csa2_kv* kv, const csa2_rows* rows, const void* q_idx, csa2_dtype q_dtype,
                             int32_t n_idx_heads, const float* w, const int32_t* pool_blocks, int64_t pool_stride,
                             const int32_t* pool_count, float* scores, int64_t scores_stride, float* block_max,
                             int64_t block_max_stride, void* stream) {
    csa2::KvView v;
    csa2_status s = make_view(kv, false, true, &v);
    if (s != CSA2_OK) return s;
    if ((s = check_rows(rows)) != CSA2_OK) return s;
    if (n_idx_heads < 1 || n_idx_heads > 64) return fail(CSA2_ERR_UNSUPPORTED, "n_idx_heads must be in 1..64 (got %d)", n_idx_heads);
    if (q_dtype != CSA2_BF16 && q_dtype != CSA2_F32) return fail(CSA2_ERR_UNSUPPORTED, "unknown q dtype");
    if (rows->n_rows == 0) return CSA2_OK;
    if (!q_idx || !w) return fail(CSA2_ERR_NULL, "q_idx / w is NULL");
    if (!aligned(q_idx, 16)) return fail(CSA2_ERR_ALIGN, "q_idx must be 16-byte aligned");
    if (pool_blocks) {
        if (!pool_count) return fail(CSA2_ERR_NULL, "pool mode needs pool_count");
        if (pool_stride < 1) return fail(CSA2_ERR_SHAPE, "pool_stride must be >= 1");
        if (block_max) return fail(CSA2_ERR_SHAPE, "block_max must be NULL in pool mode");
        if (!scores) return fail(CSA2_ERR_NULL, "pool mode needs scores");
        if (scores_stride < 8 * (int64_t)(pool_stride < 2048 ? pool_stride : 2048))
            return fail(CSA2_ERR_SHAPE, "scores_stride must cover 8 columns per pool block");
    } else {
        if (!scores && !block_max) return fail(CSA2_ERR_NULL, "scores and block_max are both NULL");
        const int64_t nv8 = ((int64_t)rows->max_vis + 7) & ~(int64_t)7;
        if (scores && scores_stride < nv8) return fail(CSA2_ERR_SHAPE, "scores_stride %lld < roundup(max_vis, 8)", (long long)scores_stride);
        if (block_max && block_max_stride < nv8 / 8) return fail(CSA2_ERR_SHAPE, "block_max_stride too small");
        if (rows->max_vis == 0) return CSA2_OK;
    }
    csa2::IndexScoreArgs a;
    a.q_idx = q_idx;
    a.q_bf16 = q_dtype == CSA2_BF16;
    a.n_heads = n_idx_heads;
    a.w = w;
    a.req = rows->req;
    a.n_vis = rows->n_vis;
    a.n_rows = rows->n_rows;
    a.max_vis = rows->max_vis;
    a.pool = pool_blocks;
    a.pool_stride = pool_stride;
    a.pool_count = pool_count;
    a.scores = scores;
    a.scores_stride = scores_stride;
    a.block_max = block_max;
    a.block_max_stride = block_max_stride;
    return hip_status(csa2::launch_index_score(v, a, (hipStream_t)stream), "csa2_index_score launch");
}

csa2_status csa2_index_score_shared(const csa2_kv* kv, const csa2_rows* rows, int32_t req, const void* q_idx,
                                    csa2_dtype q_dtype, int32_t n_idx_heads, const float* w, float* scores,
                                    int64_t scores_stride, float* block_max, int64_t block_max_stride, void* stream) {
    csa2::KvView v;
    csa2_status s = make_view(kv, false, true, &v);
    if (s != CSA2_OK) return s;
    if (!rows) return fail(CSA2_ERR_NULL, "rows descriptor is NULL");
    if (rows->n_rows < 0 || rows->n_rows > 65535) return fail(CSA2_ERR_RANGE, "n_rows must be in 0..65535");
    if (rows->max_vis < 0 || rows->max_vis > (1 << 30)) return fail(CSA2_ERR_RANGE, "max_vis out of range");
    if (n_idx_heads < 1 || n_idx_heads > 16) return fail(CSA2_ERR_UNSUPPORTED, "n_idx_heads must be in 1..16 (got %d)", n_idx_heads);
    if (q_dtype != CSA2_BF16 && q_dtype != CSA2_F32) return fail(CSA2_ERR_UNSUPPORTED, "unknown q dtype");
    if (req < 0) return fail(CSA2_ERR_RANGE, "req must be >= 0");
    if (rows->n_rows == 0) return CSA2_OK;
    if (!rows->n_vis) return fail(CSA2_ERR_NULL, "rows->n_vis is NULL");
    if (!q_idx || !w) return fail(CSA2_ERR_NULL, "q_idx / w is NULL");
    if (!aligned(q_idx, 16)) return fail(CSA2_ERR_ALIGN, "q_idx must be 16-byte aligned");
    if (!scores && !block_max) return fail(CSA2_ERR_NULL, "scores and block_max are both NULL");
    const int64_t nv8 = ((int64_t)rows->max_vis + 7) & ~(int64_t)7;
    if (scores && scores_stride < nv8) return fail(CSA2_ERR_SHAPE, "scores_stride %lld < roundup(max_vis, 8)", (long long)scores_stride);
    if (block_max && block_max_stride < nv8 / 8) return fail(CSA2_ERR_SHAPE, "block_max_stride too small");
    if (rows->max_vis == 0) return CSA2_OK;
    csa2::IndexScoreArgs a;
    a.q_idx = q_idx;
    a.q_bf16 = q_dtype == CSA2_BF16;
    a.n_heads = n_idx_heads;
    a.w = w;
    a.req = nullptr;
    a.n_vis = rows->n_vis;
    a.n_rows = rows->n_rows;
    a.max_vis = rows->max_vis;
    a.pool = nullptr;
    a.pool_stride = 0;
    a.pool_count = nullptr;
    a.scores = scores;
    a.scores_stride = scores_stride;
    a.block_max = block_max;
    a.block_max_stride = block_max_stride;
    return hip_status(csa2::launch_index_score_shared(v, a, req, (hipStream_t)stream), "csa2_index_score_shared launch");
}

size_t csa2_select_topk_workspace(int32_t n_rows, int32_t max_cols, int32_t k) {
    (void)n_rows;
    (void)max_cols;
    (void)k;
    return 0;   // the selection lives in LDS and registers
}

csa2_status csa2_select_topk(const float* keys, int64_t key_stride, const int32_t* ids, int64_t ids_stride,
                             const int32_t* n_cols, int32_t cols_mul, int32_t cols_div, const int32_t* pool_blocks,
                             int64_t pool_stride, int32_t keys_by_id, int32_t n_rows, int32_t max_cols, int32_t k,
                             int32_t* out_ids, int64_t out_stride, int32_t* out_count, void* workspace,
                             size_t workspace_bytes, void* stream) {
    if (n_rows < 0 || n_rows > 65535) return fail(CSA2_ERR_RANGE, "n_rows out of range");
    if (workspace_bytes && !workspace) return fail(CSA2_ERR_NULL, "workspace_bytes > 0 with a NULL workspace");
    if (workspace && !aligned(workspace, 256)) return fail(CSA2_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (k < 1 || k > CSA2_MAX_SELECT) return fail(CSA2_ERR_RANGE, "k must be in 1..%d (got %d)", CSA2_MAX_SELECT, k);
    if (max_cols < 0 || max_cols > (1 << 24)) return fail(CSA2_ERR_RANGE, "max_cols out of range");
    if (cols_mul < 1 || cols_mul > 8 || cols_div < 1 || cols_div > 8) return fail(CSA2_ERR_RANGE, "cols_mul / cols_div must be in 1..8");
    if (n_rows == 0) return CSA2_OK;
    if (!keys || !out_ids || !out_count) return fail(CSA2_ERR_NULL, "keys / out_ids / out_count is NULL");
    if (out_stride < k) return fail(CSA2_ERR_SHAPE, "out_stride < k");
    if (keys_by_id && !pool_blocks) return fail(CSA2_ERR_SHAPE, "keys_by_id needs pool_blocks");
    if (keys_by_id && (!aligned(keys, 16) || key_stride % 4))
        return fail(CSA2_ERR_ALIGN, "keys_by_id needs 16-byte aligned keys and key_stride % 4 == 0");
    if (pool_blocks && pool_stride < 1) return fail(CSA2_ERR_SHAPE, "pool_stride must be >= 1");
    if (ids && pool_blocks) return fail(CSA2_ERR_SHAPE, "ids and pool_blocks are exclusive");
    if (ids && ids_stride < max_cols) return fail(CSA2_ERR_SHAPE, "ids_stride < max_cols");
    if (!keys_by_id && key_stride < max_cols) return fail(CSA2_ERR_SHAPE, "key_stride < max_cols");
    if (pool_blocks && (int64_t)max_cols > 8 * pool_stride) return fail(CSA2_ERR_SHAPE, "max_cols exceeds 8 * pool_stride");
    csa2::TopkArgs a;
    a.keys = keys;
    a.key_stride = key_stride;
    a.ids = ids;
    a.ids_stride = ids_stride;
    a.n_cols = n_cols;
    a.cols_mul = cols_mul;
    a.cols_div = cols_div;
    a.pool = pool_blocks;
    a.pool_stride = pool_stride;
    a.keys_by_id = keys_by_id != 0;
    a.n_rows = n_rows;
    a.max_cols = max_cols;
    a.k = k;
    a.out_ids = out_ids;
    a.out_stride = out_stride;
    a.out_count = out_count;
    return hip_status(csa2::launch_topk(a, (hipStream_t)stream), "csa2_select_topk launch");
}

size_t csa2_attn_workspace_size(int32_t n_rows, int32_t n_heads) {
    if (n_rows <= 0 || n_heads < 16 || n_heads > 128) return 0;
    return csa2::attn_workspace_bytes(n_rows, n_heads, csa2::attn_splits(n_rows, n_heads));
}

static csa2_status check_heads(int32_t h) {
    if (!(h == 16 || h == 32 || h == 48 || h == 64 || h == 128))
        return fail(CSA2_ERR_UNSUPPORTED, "n_heads must be 16, 32, 48, 64 or 128 (got %d)", h);
    return CSA2_OK;
}

static csa2_status check_common(int32_t n_rows, const void* q, csa2_dtype q_dtype, int32_t n_heads, float scale,
                                const void* workspace) {
    csa2_status s = check_heads(n_heads);
    if (s != CSA2_OK) return s;
    if (n_rows < 0 || n_rows > 65535) return fail(CSA2_ERR_RANGE, "n_rows out of range");
    if (q_dtype != CSA2_BF16 && q_dtype != CSA2_F32) return fail(CSA2_ERR_UNSUPPORTED, "unknown q dtype");
    if (n_rows == 0) return CSA2_OK;
    if (!q) return fail(CSA2_ERR_NULL, "q is NULL");
    if (!aligned(q, 16)) return fail(CSA2_ERR_ALIGN, "q must be 16-byte aligned");
    if (!(scale > 0.0f) || scale > 1e30f) return fail(CSA2_ERR_RANGE, "softmax_scale must be positive and finite");
    if (workspace && !aligned(workspace, 256)) return fail(CSA2_ERR_ALIGN, "workspace must be 256-byte aligned");
    return CSA2_OK;
}

static csa2_status check_swa(const uint8_t* codes, const uint8_t* scales, int64_t slots, const int64_t* first,
                             const int32_t* count) {
    if (!codes || !scales || !first || !count) return fail(CSA2_ERR_NULL, "SWA planes / swa_first / swa_count is NULL");
    if (!aligned(codes, 256) || !aligned(scales, 256)) return fail(CSA2_ERR_ALIGN, "SWA planes must be 256-byte aligned");
    if (slots <= 0) return fail(CSA2_ERR_RANGE, "swa_slots must be positive");
    return CSA2_OK;
}

static void fill_q(csa2::AttnArgs& a, const void* q, csa2_dtype q_dtype, int32_t n_heads, int32_t n_rows, float scale,
                   void* workspace) {
    memset(&a, 0, sizeof a);
    a.q = q;
    a.q_bf16 = q_dtype == CSA2_BF16;
    a.n_heads = n_heads;
    a.n_rows = n_rows;
    a.scale = scale;
    a.ws = (float*)workspace;
}

csa2_status csa2_select_full(const float* block_max, int64_t block_max_stride, const float* scores,
                             int64_t scores_stride, const int32_t* n_vis, int32_t n_rows, int32_t max_vis,
                             int32_t n_pool_blocks, int32_t k, int32_t* pool, int64_t pool_stride,
                             int32_t* pool_count, int32_t* idx, int64_t idx_stride, int32_t* idx_count,
                             void* stream) {
    if (n_rows < 0 || n_rows > 65535) return fail(CSA2_ERR_RANGE, "n_rows out of range");
    if (max_vis < 0 || max_vis > (1 << 24)) return fail(CSA2_ERR_RANGE, "max_vis out of range");
    if (n_pool_blocks < 1 || n_pool_blocks > CSA2_MAX_POOL_BLOCKS)
        return fail(CSA2_ERR_RANGE, "n_pool_blocks must be in 1..%d (got %d)", CSA2_MAX_POOL_BLOCKS, n_pool_blocks);
    if (k < 1 || k > CSA2_MAX_SELECT) return fail(CSA2_ERR_RANGE, "k must be in 1..%d (got %d)", CSA2_MAX_SELECT, k);
    if (n_rows == 0) return CSA2_OK;
    if (!block_max || !scores || !n_vis || !pool || !pool_count || !idx || !idx_count)
        return fail(CSA2_ERR_NULL, "a required pointer is NULL");
    const int64_t nv8 = ((int64_t)max_vis + 7) & ~(int64_t)7;
    if (block_max_stride < nv8 / 8) return fail(CSA2_ERR_SHAPE, "block_max_stride < ceil(max_vis / 8)");
    if (scores_stride < nv8) return fail(CSA2_ERR_SHAPE, "scores_stride < roundup(max_vis, 8)");
    if (pool_stride < n_pool_blocks) return fail(CSA2_ERR_SHAPE, "pool_stride < n_pool_blocks");
    if (idx_stride < k) return fail(CSA2_ERR_SHAPE, "idx_stride < k");
    if (!aligned(scores, 16) || scores_stride % 4) return fail(CSA2_ERR_ALIGN, "scores rows must be 16-byte aligned");
    csa2::SelectFullArgs a;
    a.block_max = block_max;
    a.block_max_stride = block_max_stride;
    a.scores = scores;
    a.scores_stride = scores_stride;
    a.n_vis = n_vis;
    a.n_rows = n_rows;
    a.max_vis = max_vis;
    a.n_pool = n_pool_blocks;
    a.k = k;
    a.pool = pool;
    a.pool_stride = pool_stride;
    a.pool_count = pool_count;
    a.idx = idx;
    a.idx_stride = idx_stride;
    a.idx_count = idx_count;
    return hip_status(csa2::launch_select_full(a, (hipStream_t)stream), "csa2_select_full launch");
}

csa2_status csa2_sparse_attn(const csa2_kv* kv, const csa2_rows* rows, const void* q, csa2_dtype q_dtype,
                             int32_t n_heads, const int32_t* idx, int64_t idx_stride, const int32_t* idx_count,
                             float softmax_scale, float* o_partial, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
    csa2::KvView v;
    csa2_status s = make_view(kv, true, false, &v);
    if (s != CSA2_OK) return s;
    if ((s = check_rows(rows)) != CSA2_OK) return s;
    if ((s = check_common(rows->n_rows, q, q_dtype, n_heads, softmax_scale, workspace)) != CSA2_OK) return s;
    if (rows->n_rows == 0) return CSA2_OK;
    if (!idx || !idx_count || !o_partial || !lse) return fail(CSA2_ERR_NULL, "idx / idx_count / o_partial / lse is NULL");
    if (!aligned(o_partial, 16)) return fail(CSA2_ERR_ALIGN, "o_partial must be 16-byte aligned");
    if (idx_stride < 1) return fail(CSA2_ERR_SHAPE, "idx_stride must be >= 1");
    csa2::AttnArgs a;
    fill_q(a, q, q_dtype, n_heads, rows->n_rows, softmax_scale, workspace);
    a.req = rows->req;
    a.idx = idx;
    a.idx_stride = idx_stride;
    a.idx_count = idx_count;
    a.out = o_partial;
    a.lse_out = lse;
    return hip_status(csa2::launch_attn(v, a, workspace_bytes, (hipStream_t)stream), "csa2_sparse_attn launch");
}

csa2_status csa2_swa_merge(const uint8_t* swa_codes, const uint8_t* swa_scales, int64_t swa_slots,
                           const int64_t* swa_first, const int32_t* swa_count, int32_t n_rows, const void* q,
                           csa2_dtype q_dtype, int32_t n_heads, float softmax_scale, const float* sink,
                           const float* o_partial, const float* lse, float* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
    csa2_status s = check_common(n_rows, q, q_dtype, n_heads, softmax_scale, workspace);
    if (s != CSA2_OK) return s;
    if (n_rows == 0) return CSA2_OK;
    if ((s = check_swa(swa_codes, swa_scales, swa_slots, swa_first, swa_count)) != CSA2_OK) return s;
    if (!out) return fail(CSA2_ERR_NULL, "out is NULL");
    if ((o_partial == nullptr) != (lse == nullptr)) return fail(CSA2_ERR_NULL, "o_partial and lse must be both set or both NULL");
    if (!aligned(out, 16) || (o_partial && !aligned(o_partial, 16))) return fail(CSA2_ERR_ALIGN, "out and o_partial must be 16-byte aligned");
    csa2::AttnArgs a;
    fill_q(a, q, q_dtype, n_heads, n_rows, softmax_scale, workspace);
    a.swa_codes = swa_codes;
    a.swa_scales = swa_scales;
    a.swa_first = swa_first;
    a.swa_count = swa_count;
    a.sink = sink;
    a.o_in = o_partial;
    a.lse_in = lse;
    a.out = out;
    csa2::KvView none;
    memset(&none, 0, sizeof none);
    return hip_status(csa2::launch_attn(none, a, workspace_bytes, (hipStream_t)stream), "csa2_swa_merge launch");
}

static csa2_status sparse_swa_args(const csa2_kv* kv, const csa2_rows* rows, const void* q, csa2_dtype q_dtype,
                                   int32_t n_heads, const int32_t* idx, int64_t idx_stride, const int32_t* idx_count,
                                   const uint8_t* swa_codes, const uint8_t* swa_scales, int64_t swa_slots,
                                   const int64_t* swa_first, const int32_t* swa_count, const float* sink,
                                   float softmax_scale, float* out, float* lse, void* workspace, csa2::KvView* v,
                                   csa2::AttnArgs* a) {
    csa2_status s = make_view(kv, true, false, v);
    if (s != CSA2_OK) return s;
    if ((s = check_rows(rows)) != CSA2_OK) return s;
    if ((s = check_common(rows->n_rows, q, q_dtype, n_heads, softmax_scale, workspace)) != CSA2_OK) return s;
    if (rows->n_rows == 0) return CSA2_OK;
    if ((s = check_swa(swa_codes, swa_scales, swa_slots, swa_first, swa_count)) != CSA2_OK) return s;
    if (!idx || !idx_count || !out) return fail(CSA2_ERR_NULL, "idx / idx_count / out is NULL");
    if (!aligned(out, 16)) return fail(CSA2_ERR_ALIGN, "out must be 16-byte aligned");
    if (idx_stride < 1) return fail(CSA2_ERR_SHAPE, "idx_stride must be >= 1");
    fill_q(*a, q, q_dtype, n_heads, rows->n_rows, softmax_scale, workspace);
    a->req = rows->req;
    a->idx = idx;
    a->idx_stride = idx_stride;
    a->idx_count = idx_count;
    a->swa_codes = swa_codes;
    a->swa_scales = swa_scales;
    a->swa_first = swa_first;
    a->swa_count = swa_count;
    a->sink = sink;
    a->out = out;
    a->lse_out = lse;
    return CSA2_OK;
}

csa2_status csa2_sparse_swa_attn(const csa2_kv* kv, const csa2_rows* rows, const void* q, csa2_dtype q_dtype,
                                 int32_t n_heads, const int32_t* idx, int64_t idx_stride, const int32_t* idx_count,
                                 const uint8_t* swa_codes, const uint8_t* swa_scales, int64_t swa_slots,
                                 const int64_t* swa_first, const int32_t* swa_count, const float* sink,
                                 float softmax_scale, float* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    csa2::KvView v;
    csa2::AttnArgs a;
    csa2_status s = sparse_swa_args(kv, rows, q, q_dtype, n_heads, idx, idx_stride, idx_count, swa_codes, swa_scales,
                                    swa_slots, swa_first, swa_count, sink, softmax_scale, out, lse, workspace, &v, &a);
    if (s != CSA2_OK || rows->n_rows == 0) return s;
    return hip_status(csa2::launch_attn(v, a, workspace_bytes, (hipStream_t)stream), "csa2_sparse_swa_attn launch");
}

csa2_status csa2_sparse_swa_attn_noalloc(const csa2_kv* kv, const csa2_rows* rows, const void* q, csa2_dtype q_dtype,
                                         int32_t n_heads, const int32_t* idx, int64_t idx_stride,
                                         const int32_t* idx_count, const uint8_t* swa_codes,
                                         const uint8_t* swa_scales, int64_t swa_slots, const int64_t* swa_first,
                                         const int32_t* swa_count, const float* sink, float softmax_scale,
                                         float* out, float* lse, void* stream) {
    csa2::KvView v;
    csa2::AttnArgs a;
    csa2_status s = sparse_swa_args(kv, rows, q, q_dtype, n_heads, idx, idx_stride, idx_count, swa_codes, swa_scales,
                                    swa_slots, swa_first, swa_count, sink, softmax_scale, out, lse, nullptr, &v, &a);
    if (s != CSA2_OK || rows->n_rows == 0) return s;
    const size_t need = csa2_attn_workspace_size(rows->n_rows, n_heads);
    if (need > CSA2_ATTN_SCRATCH_BYTES)
        return fail(CSA2_ERR_RANGE, "csa2_sparse_swa_attn_noalloc: the split pass of %d rows x %d heads needs %zu "
                                    "bytes of scratch, more than the %zu the library holds",
                    rows->n_rows, n_heads, need, (size_t)CSA2_ATTN_SCRATCH_BYTES);
    if (need == 0) return hip_status(csa2::launch_attn(v, a, 0, (hipStream_t)stream), "csa2_sparse_swa_attn_noalloc launch");
    void* ptr = nullptr;
    size_t bytes = 0;
    hipError_t e = csa2::noalloc_scratch(&ptr, &bytes);
    if (e != hipSuccess) return hip_status(e, "csa2_sparse_swa_attn_noalloc: scratch address");
    a.ws = (float*)ptr;
    return hip_status(csa2::launch_attn(v, a, need, (hipStream_t)stream), "csa2_sparse_swa_attn_noalloc launch");
}

size_t csa2_dense_attn_workspace_size(int32_t n_rows, int32_t n_heads, int32_t max_vis) {
    if (n_rows <= 0 || n_heads < 16 || n_heads > 128 || max_vis < 0 || max_vis > CSA2_MAX_DENSE) return 0;
    return csa2::dense_workspace_bytes(n_rows, n_heads, max_vis);
}

csa2_status csa2_dense_swa_attn(const csa2_kv* kv, const csa2_rows* rows, const void* q, csa2_dtype q_dtype,
                                int32_t n_heads, const uint8_t* swa_codes, const uint8_t* swa_scales,
                                int64_t swa_slots, const int64_t* swa_first, const int32_t* swa_count,
                                const float* sink, float softmax_scale, float* out, float* lse, void* workspace,
                                size_t workspace_bytes, void* stream) {
    csa2::KvView v;
    csa2_status s = make_view(kv, true, false, &v);
    if (s != CSA2_OK) return s;
    if ((s = check_rows(rows)) != CSA2_OK) return s;
    if ((s = check_common(rows->n_rows, q, q_dtype, n_heads, softmax_scale, workspace)) != CSA2_OK) return s;
    if (rows->max_vis > CSA2_MAX_DENSE)
        return fail(CSA2_ERR_RANGE, "max_vis %d above %d entries", rows->max_vis, CSA2_MAX_DENSE);
    if (rows->n_rows == 0) return CSA2_OK;
    if (swa_codes && (s = check_swa(swa_codes, swa_scales, swa_slots, swa_first, swa_count)) != CSA2_OK) return s;
    if (!out) return fail(CSA2_ERR_NULL, "out is NULL");
    if (!aligned(out, 16)) return fail(CSA2_ERR_ALIGN, "out must be 16-byte aligned");
    csa2::AttnArgs a;
    fill_q(a, q, q_dtype, n_heads, rows->n_rows, softmax_scale, workspace);
    a.req = rows->req;
    a.dense_n = rows->n_vis;
    a.max_dense = rows->max_vis;
    if (swa_codes) {
        a.swa_codes = swa_codes;
        a.swa_scales = swa_scales;
        a.swa_first = swa_first;
        a.swa_count = swa_count;
    }
    a.sink = sink;
    a.out = out;
    a.lse_out = lse;
    return hip_status(csa2::launch_attn_dense(v, a, workspace_bytes, (hipStream_t)stream), "csa2_dense_swa_attn launch");
}

csa2_status csa2_synth_normal(uint64_t seed, uint32_t tensor_id, int64_t first, int64_t n, csa2_dtype out_dtype,
                              void* out, void* stream) {
    if (n < 0 || first < 0) return fail(CSA2_ERR_RANGE, "first / n must be >= 0");
    if (n == 0) return CSA2_OK;
    if (!out) return fail(CSA2_ERR_NULL, "out is NULL");
    if (out_dtype != CSA2_BF16 && out_dtype != CSA2_F32) return fail(CSA2_ERR_UNSUPPORTED, "unknown dtype");
    if (n > ((int64_t)1 << 38)) return fail(CSA2_ERR_RANGE, "n too large for one call");
    return hip_status(csa2::launch_synth_normal(seed, tensor_id, first, n, out_dtype == CSA2_BF16, out, (hipStream_t)stream),
                      "csa2_synth_normal launch");
}

csa2_status csa2_stream_xor(const void* buf, int64_t n_bytes, uint32_t* out, void* stream) {
    if (n_bytes < 0) return fail(CSA2_ERR_RANGE, "n_bytes must be >= 0");
    if (n_bytes % 16) return fail(CSA2_ERR_SHAPE, "n_bytes must be a multiple of 16");
    if (n_bytes == 0) return CSA2_OK;
    if (!buf || !out) return fail(CSA2_ERR_NULL, "buf / out is NULL");
    if (!aligned(buf, 16) || !aligned(out, 4)) return fail(CSA2_ERR_ALIGN, "buf must be 16-B and out 4-B aligned");
    return hip_status(csa2::launch_stream_xor(buf, n_bytes, out, (hipStream_t)stream), "csa2_stream_xor launch");
}

csa2_status csa2_synth_uniform(uint64_t seed, uint32_t tensor_id, int64_t first, int64_t n, float* out, void* stream) {
    if (n < 0 || first < 0) return fail(CSA2_ERR_RANGE, "first / n must be >= 0");
    if (n == 0) return CSA2_OK;
    if (!out) return fail(CSA2_ERR_NULL, "out is NULL");
    if (n > ((int64_t)1 << 38)) return fail(CSA2_ERR_RANGE, "n too large for one call");
    return hip_status(csa2::launch_synth_uniform(seed, tensor_id, first, n, out, (hipStream_t)stream), "csa2_synth_uniform launch");
}

csa2_status csa2_synth_boost(uint64_t seed, uint32_t boost_tensor, int64_t first_pos, int64_t n_rows, int32_t width,
                             float* x, void* stream) {
    if (n_rows < 0 || first_pos < 0 || width < 1) return fail(CSA2_ERR_RANGE, "bad sizes");
    if (n_rows == 0) return CSA2_OK;
    if (!x) return fail(CSA2_ERR_NULL, "x is NULL");
    if (n_rows * (int64_t)width > ((int64_t)1 << 38)) return fail(CSA2_ERR_RANGE, "too large for one call");
    return hip_status(csa2::launch_synth_boost(seed, boost_tensor, first_pos, n_rows, width, x, (hipStream_t)stream),
                      "csa2_synth_boost launch");
}

}  // extern "C"
