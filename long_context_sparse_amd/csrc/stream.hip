// stream.hip -- the plain streaming read that the indexer scan's HBM rate is
// compared with (not a step of the method).  Every 16-B word of a buffer is
// read once with a non-temporal load, as the scan reads its keys, by a fixed
// grid of 1,024 workgroups striding over the buffer (the fastest of grids
// of 1,024 to 16,384 workgroups with 2, 4 or 8 loads in flight per lane).  Workgroup g writes the
// XOR of the 32-bit words it read to out[g] (one plain store; atomics on one
// shared word would serialise thousands of waves at the end), so the loads
// cannot be dropped and the XOR of the 1,024 words checks the read.
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

typedef unsigned int sx_u32x4 __attribute__((ext_vector_type(4)));
constexpr int SX_THREADS = 256;
constexpr int SX_UNROLL = 2;                 // loads in flight per lane
constexpr int SX_GRID = 1024;                // 4 workgroups per CU; one output word each

__global__ __launch_bounds__(SX_THREADS) void stream_xor_kernel(const sx_u32x4* __restrict__ p, int64_t n16,
                                                                uint32_t* out) {
    __shared__ uint32_t wx[SX_THREADS / 64];
    const int64_t stride = (int64_t)gridDim.x * SX_THREADS;
    int64_t i = (int64_t)blockIdx.x * SX_THREADS + threadIdx.x;
    uint32_t acc = 0u;
    for (; i + (SX_UNROLL - 1) * stride < n16; i += SX_UNROLL * stride) {
        sx_u32x4 v[SX_UNROLL];
#pragma unroll
        for (int u = 0; u < SX_UNROLL; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < SX_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const sx_u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, d, 64);
    if ((threadIdx.x & 63) == 0) wx[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0u;
#pragma unroll
        for (int w = 0; w < SX_THREADS / 64; ++w) x ^= wx[w];
        out[blockIdx.x] = x;
    }
}

hipError_t launch_stream_xor(const void* buf, int64_t n_bytes, uint32_t* out, hipStream_t st) {
    // every workgroup writes its word, also those with nothing to read
    hipLaunchKernelGGL(stream_xor_kernel, dim3(SX_GRID), dim3(SX_THREADS), 0, st, (const sx_u32x4*)buf, n_bytes / 16, out);
    return hipGetLastError();
}

}  // namespace csa2
