// csa2_launch.h -- internal launchers of the CSA2 kernels, called by the
// C-ABI layer (api.cpp) after it has validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

struct KvView;

hipError_t launch_pack(int kind, const void* src, bool bf16, int64_t n, int64_t stride,
                       uint8_t* codes, uint8_t* scales, const int64_t* slots, hipStream_t st);

struct IndexScoreArgs {
    const void* q_idx;
    bool q_bf16;
    int n_heads;
    const float* w;
    const int32_t* req;
    const int32_t* n_vis;
    int n_rows;
    int max_vis;
    const int32_t* pool;      // NULL: full scan
    int64_t pool_stride;
    const int32_t* pool_count;
    float* scores;
    int64_t scores_stride;
    float* block_max;
    int64_t block_max_stride;
};
hipError_t launch_index_score(const KvView& kv, const IndexScoreArgs& a, hipStream_t st);
// rows 0 .. n_rows-1 all read request `req` (full scan only; a.req is not read)
hipError_t launch_index_score_shared(const KvView& kv, const IndexScoreArgs& a, int req, hipStream_t st);

struct TopkArgs {
    const float* keys;
    int64_t key_stride;
    const int32_t* ids;           // id per column (NULL: column index or pool position)
    int64_t ids_stride;
    const int32_t* n_cols;
    int cols_mul, cols_div;
    const int32_t* pool;
    int64_t pool_stride;
    bool keys_by_id;
    int n_rows, max_cols, k;
    int32_t* out_ids;
    int64_t out_stride;
    int32_t* out_count;
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);

// The Full layer's two selections in one pass per row: the pool (top n_pool
// blocks by block maximum) and the top k positions among the pool's scores.
struct SelectFullArgs {
    const float* block_max;
    int64_t block_max_stride;
    const float* scores;          // 16-B aligned rows, -inf past n_vis up to a multiple of 8
    int64_t scores_stride;
    const int32_t* n_vis;
    int n_rows, max_vis, n_pool, k;
    int32_t* pool;
    int64_t pool_stride;
    int32_t* pool_count;
    int32_t* idx;
    int64_t idx_stride;
    int32_t* idx_count;
};
hipError_t launch_select_full(const SelectFullArgs& a, hipStream_t st);

// Joint attention over a row's selected FP4 entries (idx) and its 8-bit
// window (swa_*), plus an optional external partial (o_in, lse_in) and sink.
struct AttnArgs {
    const void* q;
    bool q_bf16;
    int n_heads;
    const int32_t* req;
    int n_rows;
    const int32_t* idx;          // NULL: no selected entries
    int64_t idx_stride;
    const int32_t* idx_count;
    const uint8_t* swa_codes;    // NULL: no window
    const uint8_t* swa_scales;
    const int64_t* swa_first;
    const int32_t* swa_count;
    float scale;
    const float* sink;
    const float* o_in;
    const float* lse_in;
    float* out;
    float* lse_out;
    float* ws;                   // split partials (NULL: one workgroup per row and head group)
    int n_splits;                // set by the launchers
    int max_units;               // unit slots per (row, head) in ws; set by the launchers
    const int32_t* dense_n;      // dense rows: entries [0, dense_n[row]) of the row (launch_attn_dense)
    int max_dense;               // bound on dense_n
};
int attn_splits(int n_rows, int n_heads);
size_t attn_workspace_bytes(int n_rows, int n_heads, int n_splits);
hipError_t launch_attn(const KvView& kv, const AttnArgs& a, size_t ws_bytes, hipStream_t st);
// Every visible entry of each row instead of a selection (the heavily
// compressed branch): a.dense_n / a.max_dense give the rows' entry counts.
int dense_units(int max_dense);
size_t dense_workspace_bytes(int n_rows, int n_heads, int max_dense);
hipError_t launch_attn_dense(const KvView& kv, const AttnArgs& a, size_t ws_bytes, hipStream_t st);

// Address (on the current device) and size of the library's own scratch
// array for the allocation-free attention; looked up once per device.
hipError_t noalloc_scratch(void** out, size_t* bytes);

// The write path: compressed entries from projected token streams, then
// RMSNorm, RoPE and packing (MAIN width 512 or INDEX width 128).
struct CompressArgs {
    int m;                       // tokens per block
    const float* ca;             // value / logit streams of the entry's own block, token rows of `stride`
    const float* za;
    const float* cb;             // of the block before (NULL: no overlap)
    const float* zb;
    const float* ba;             // positional biases [m][width]
    const float* bb;
    int64_t stride;
    int64_t n_ent;               // entries = complete blocks
    const float* norm_weight;    // [width] or NULL: no RMSNorm
    float eps;
    int rope;                    // rotate the last 64 channels
    int64_t pos0;                // token position of entry 0
    double inv_freq[32];         // 10000^(-2j/64), j = 0 .. 31 (set by the launcher)
};
hipError_t launch_compress_pack(const CompressArgs& a, int width, float* values, uint8_t* codes, uint8_t* scales,
                                const int64_t* slots, hipStream_t st);

hipError_t launch_stream_xor(const void* buf, int64_t n_bytes, uint32_t* out, hipStream_t st);

hipError_t launch_synth_normal(uint64_t seed, uint32_t tensor, int64_t first, int64_t n, bool bf16,
                               void* out, hipStream_t st);
hipError_t launch_synth_uniform(uint64_t seed, uint32_t tensor, int64_t first, int64_t n, float* out,
                                hipStream_t st);
hipError_t launch_synth_boost(uint64_t seed, uint32_t tensor, int64_t first_pos, int64_t n_rows, int width,
                              float* x, hipStream_t st);

}  // namespace csa2
