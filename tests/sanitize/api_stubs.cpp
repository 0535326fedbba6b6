// api_stubs.cpp -- host-only stand-ins for the kernel launchers of libcsa2,
// so that the C ABI's argument validation (api.cpp) can be built and driven
// on a machine without a GPU under the host sanitizers.  Every launcher
// records that it was reached and returns success; the workspace helpers
// return fixed sizes.
#include <hip/hip_runtime.h>

#include "../../long_context_sparse_amd/csrc/csa2_launch.h"

int g_launches = 0;

namespace csa2 {
hipError_t launch_pack(int, const void*, bool, int64_t, int64_t, uint8_t*, uint8_t*, const int64_t*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_index_score(const KvView&, const IndexScoreArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_index_score_shared(const KvView&, const IndexScoreArgs&, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_topk(const TopkArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_select_full(const SelectFullArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
int attn_splits(int n_rows, int n_heads) { return n_rows * (n_heads / 16) <= 64 ? 4 : 1; }
size_t attn_workspace_bytes(int n_rows, int n_heads, int n_splits) { return n_splits > 1 ? (size_t)n_rows * n_heads * 4 * 514 * 4 : 0; }
hipError_t launch_attn(const KvView&, const AttnArgs&, size_t, hipStream_t) { ++g_launches; return hipSuccess; }
int dense_units(int max_dense) { return (max_dense + 63) / 64 / 3 + 1; }
size_t dense_workspace_bytes(int n_rows, int n_heads, int max_dense) { return (size_t)n_rows * n_heads * dense_units(max_dense) * 514 * 4; }
hipError_t launch_attn_dense(const KvView&, const AttnArgs&, size_t, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t noalloc_scratch(void** out, size_t* bytes) { static char buf[256]; *out = buf; *bytes = sizeof buf; return hipSuccess; }
hipError_t launch_compress_pack(const CompressArgs&, int, float*, uint8_t*, uint8_t*, const int64_t*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_stream_xor(const void*, int64_t, uint32_t*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_synth_normal(uint64_t, uint32_t, int64_t, int64_t, bool, void*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_synth_uniform(uint64_t, uint32_t, int64_t, int64_t, float*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_synth_boost(uint64_t, uint32_t, int64_t, int64_t, int, float*, hipStream_t) { ++g_launches; return hipSuccess; }
}  // namespace csa2
