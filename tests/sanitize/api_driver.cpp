// api_driver.cpp -- drives every entry point of the C ABI (include/csa2.h)
// with invalid and valid arguments against the launcher stand-ins of
// api_stubs.cpp, built with the host address and undefined-behaviour
// sanitizers: status codes and messages are checked, launches counted.
// Exit status 0 = clean.
#include <cstdio>
#include <cstring>

#include "../../include/csa2.h"

extern int g_launches;
static int fails = 0;
#define CHECK(c) do { if (!(c)) { std::fprintf(stderr, "check failed: %s (line %d): %s\n", #c, __LINE__, csa2_last_error()); ++fails; } } while (0)

alignas(256) static unsigned char dev[1 << 16];   // stands in for device memory (never dereferenced by the stubs)
#define D(off) ((void*)(dev + (off)))

int main() {
    CHECK(csa2_abi_version() == CSA2_ABI_VERSION);
    for (int s = -1; s < 9; ++s) CHECK(csa2_status_str(s) != nullptr);
    csa2_kv kv;
    std::memset(&kv, 0, sizeof kv);
    kv.main_codes = (const uint8_t*)D(0); kv.main_scales = (const uint8_t*)D(256);
    kv.idx_codes = (const uint8_t*)D(512); kv.idx_scales = (const uint8_t*)D(768);
    kv.n_slots = 1000; kv.req_stride = 1000;
    csa2_rows rows = {(const int32_t*)D(1024), (const int32_t*)D(1280), 2, 100};
    const int base = g_launches;
    // packing
    CHECK(csa2_pack_kv(CSA2_MAIN_FP4, D(0), CSA2_BF16, 4, 512, (uint8_t*)D(0), (uint8_t*)D(256), nullptr, nullptr) == CSA2_OK);
    CHECK(csa2_pack_kv((csa2_kind)9, D(0), CSA2_BF16, 4, 512, (uint8_t*)D(0), (uint8_t*)D(256), nullptr, nullptr) == CSA2_ERR_UNSUPPORTED);
    CHECK(csa2_pack_kv(CSA2_MAIN_FP4, D(2), CSA2_BF16, 4, 512, (uint8_t*)D(0), (uint8_t*)D(256), nullptr, nullptr) == CSA2_ERR_ALIGN);
    // write path
    csa2_compress_streams cs = {(const float*)D(0), (const float*)D(256), nullptr, nullptr, (const float*)D(512), nullptr, 8, 512, 4};
    CHECK(csa2_compress_pack(CSA2_MAIN_FP4, &cs, nullptr, 1e-6f, 1, 0, nullptr, (uint8_t*)D(0), (uint8_t*)D(256), nullptr, nullptr) == CSA2_OK);
    cs.m = 0;
    CHECK(csa2_compress_pack(CSA2_MAIN_FP4, &cs, nullptr, 1e-6f, 1, 0, nullptr, (uint8_t*)D(0), (uint8_t*)D(256), nullptr, nullptr) == CSA2_ERR_RANGE);
    cs.m = 4; cs.cb = (const float*)D(0);
    CHECK(csa2_compress_pack(CSA2_MAIN_FP4, &cs, nullptr, 1e-6f, 1, 0, nullptr, (uint8_t*)D(0), (uint8_t*)D(256), nullptr, nullptr) == CSA2_ERR_NULL);
    // indexer
    CHECK(csa2_index_score(&kv, &rows, D(0), CSA2_BF16, 8, (const float*)D(0), nullptr, 0, nullptr, (float*)D(0), 104, nullptr, 0, nullptr) == CSA2_OK);
    CHECK(csa2_index_score(&kv, &rows, D(0), CSA2_BF16, 65, (const float*)D(0), nullptr, 0, nullptr, (float*)D(0), 104, nullptr, 0, nullptr) == CSA2_ERR_UNSUPPORTED);
    CHECK(csa2_index_score(nullptr, &rows, D(0), CSA2_BF16, 8, (const float*)D(0), nullptr, 0, nullptr, (float*)D(0), 104, nullptr, 0, nullptr) == CSA2_ERR_NULL);
    CHECK(csa2_index_score_shared(&kv, &rows, 0, D(0), CSA2_BF16, 8, (const float*)D(0), (float*)D(0), 104, nullptr, 0, nullptr) == CSA2_OK);
    CHECK(csa2_index_score_shared(&kv, &rows, -1, D(0), CSA2_BF16, 8, (const float*)D(0), (float*)D(0), 104, nullptr, 0, nullptr) == CSA2_ERR_RANGE);
    // selection
    CHECK(csa2_select_topk_workspace(4, 1000, 512) == 0);
    CHECK(csa2_select_topk((const float*)D(0), 100, nullptr, 0, nullptr, 1, 1, nullptr, 0, 0, 4, 100, 10, (int32_t*)D(0), 16, (int32_t*)D(0), nullptr, 0, nullptr) == CSA2_OK);
    CHECK(csa2_select_topk((const float*)D(0), 100, (const int32_t*)D(0), 99, nullptr, 1, 1, nullptr, 0, 0, 4, 100, 10, (int32_t*)D(0), 16, (int32_t*)D(0), nullptr, 0, nullptr) == CSA2_ERR_SHAPE);
    CHECK(csa2_select_topk((const float*)D(0), 100, nullptr, 0, nullptr, 1, 1, nullptr, 0, 0, 4, 100, 0, (int32_t*)D(0), 16, (int32_t*)D(0), nullptr, 0, nullptr) == CSA2_ERR_RANGE);
    CHECK(csa2_select_full((const float*)D(0), 16, (const float*)D(0), 128, (const int32_t*)D(0), 4, 100, 2048, 512, (int32_t*)D(0), 2048, (int32_t*)D(0), (int32_t*)D(0), 512, (int32_t*)D(0), nullptr) == CSA2_OK);
    CHECK(csa2_select_full((const float*)D(0), 16, (const float*)D(4), 128, (const int32_t*)D(0), 4, 100, 2048, 512, (int32_t*)D(0), 2048, (int32_t*)D(0), (int32_t*)D(0), 512, (int32_t*)D(0), nullptr) == CSA2_ERR_ALIGN);
    // attention
    CHECK(csa2_attn_workspace_size(2, 64) > 0);
    CHECK(csa2_sparse_attn(&kv, &rows, D(0), CSA2_BF16, 64, (const int32_t*)D(0), 512, (const int32_t*)D(0), 0.04f, (float*)D(0), (float*)D(0), nullptr, 0, nullptr) == CSA2_OK);
    CHECK(csa2_sparse_attn(&kv, &rows, D(0), CSA2_BF16, 40, (const int32_t*)D(0), 512, (const int32_t*)D(0), 0.04f, (float*)D(0), (float*)D(0), nullptr, 0, nullptr) == CSA2_ERR_UNSUPPORTED);
    CHECK(csa2_swa_merge((const uint8_t*)D(0), (const uint8_t*)D(256), 10, (const int64_t*)D(0), (const int32_t*)D(0), 2, D(0), CSA2_BF16, 64, 0.04f, nullptr, nullptr, nullptr, (float*)D(0), nullptr, 0, nullptr) == CSA2_OK);
    CHECK(csa2_sparse_swa_attn(&kv, &rows, D(0), CSA2_BF16, 64, (const int32_t*)D(0), 512, (const int32_t*)D(0), (const uint8_t*)D(0), (const uint8_t*)D(256), 10, (const int64_t*)D(0), (const int32_t*)D(0), nullptr, 0.04f, (float*)D(0), nullptr, nullptr, 0, nullptr) == CSA2_OK);
    CHECK(csa2_sparse_swa_attn_noalloc(&kv, &rows, D(0), CSA2_BF16, 64, (const int32_t*)D(0), 512, (const int32_t*)D(0), (const uint8_t*)D(0), (const uint8_t*)D(256), 10, (const int64_t*)D(0), (const int32_t*)D(0), nullptr, 0.04f, (float*)D(0), nullptr, nullptr) == CSA2_OK);
    CHECK(csa2_dense_attn_workspace_size(2, 64, 8192) > 0);
    CHECK(csa2_dense_swa_attn(&kv, &rows, D(0), CSA2_BF16, 64, nullptr, nullptr, 0, nullptr, nullptr, nullptr, 0.04f, (float*)D(0), nullptr, nullptr, 0, nullptr) == CSA2_OK);
    CHECK(csa2_dense_swa_attn(&kv, &rows, D(0), CSA2_BF16, 64, nullptr, nullptr, 0, nullptr, nullptr, nullptr, 0.04f, (float*)D(4), nullptr, nullptr, 0, nullptr) == CSA2_ERR_ALIGN);
    // generator and streaming read
    CHECK(csa2_synth_normal(1, 2, 0, 16, CSA2_F32, D(0), nullptr) == CSA2_OK);
    CHECK(csa2_synth_uniform(1, 2, 0, 16, (float*)D(0), nullptr) == CSA2_OK);
    CHECK(csa2_synth_boost(1, 2, 0, 4, 16, (float*)D(0), nullptr) == CSA2_OK);
    CHECK(csa2_stream_xor(D(0), 4096, (uint32_t*)D(0), nullptr) == CSA2_OK);
    CHECK(csa2_stream_xor(D(0), 24, (uint32_t*)D(0), nullptr) == CSA2_ERR_SHAPE);
    const int launched = g_launches - base;
    CHECK(launched == 15);
    if (fails) { std::fprintf(stderr, "%d check(s) failed (launches %d)\n", fails, launched); return 1; }
    std::printf("api driver clean (%d launches reached the stubs)\n", launched);
    return 0;
}
