// pack.hip -- K1: quantise rows into the three cache formats (gfx950).
//
// Entry formats of the pages: main latent KV = 512 E2M1 + one E4M3 scale per
// 16 channels (288 B); indexer key = 128 E2M1 + one E8M0 scale per 32
// channels (68 B) ['DeepSeek V4.1 Flash architecture analysis', section
// "890 bytes/token"]; sliding-window KV kept in 8 bits ['KV cache diet' page,
// section "890 ... 10,324": SWA stays FP8, outside the 890 B].
//
// One thread quantises one channel group; consecutive threads take
// consecutive groups of a row, so source reads and code writes are
// contiguous across the wave.  This is the write path, outside the decode
// step.
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

template <bool BF16>
__device__ __forceinline__ void load_group(const void* src, int64_t off, int n, float* x) {
    if (BF16) {
        const uint16_t* p = (const uint16_t*)src + off;
        for (int i = 0; i < n; i += 8) {
            const uint4 v = *(const uint4*)(p + i);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[i + 2 * j] = __uint_as_float(w[j] << 16);
                x[i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
            }
        }
    } else {
        const float* p = (const float*)src + off;
        for (int i = 0; i < n; i += 4) {
            const float4 v = *(const float4*)(p + i);
            x[i] = v.x; x[i + 1] = v.y; x[i + 2] = v.z; x[i + 3] = v.w;
        }
    }
}

// MAIN: s = E4M3(fl32(amax / 6)); code = E2M1(fl32(x / s)); a zero scale
// gives zero codes.
template <bool BF16>
__global__ __launch_bounds__(256) void pack_main_kernel(const void* __restrict__ src, int64_t n,
                                                        int64_t stride, uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales,
                                                        const int64_t* __restrict__ slots) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= n * 32) return;
    const int64_t r = gid >> 5;
    const int g = (int)(gid & 31);
    float x[16];
    load_group<BF16>(src, r * stride + 16 * g, 16, x);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
    const uint32_t sc = e4m3_encode(__fdiv_rn(amax, 6.0f));
    const float s = e4m3_to_f32(sc);
    uint32_t lo = 0, hi = 0;
    if (s != 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) lo |= e2m1_encode(__fdiv_rn(x[i], s)) << (4 * i);
#pragma unroll
        for (int i = 0; i < 8; ++i) hi |= e2m1_encode(__fdiv_rn(x[8 + i], s)) << (4 * i);
    }
    const int64_t e = slots ? slots[r] : r;
    *(uint2*)(codes + e * 256 + 8 * g) = make_uint2(lo, hi);
    scales[e * 32 + g] = (uint8_t)sc;
}

// INDEX (MXFP4): e = floor(log2 amax) - 2; code = E2M1(x * 2^-e).
template <bool BF16>
__global__ __launch_bounds__(256) void pack_index_kernel(const void* __restrict__ src, int64_t n,
                                                         int64_t stride, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales,
                                                         const int64_t* __restrict__ slots) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= n * 4) return;
    const int64_t r = gid >> 2;
    const int g = (int)(gid & 3);
    float x[32];
    load_group<BF16>(src, r * stride + 32 * g, 32, x);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
    const int ex = mx_exponent(amax, 2);
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 32; ++i) w[i >> 3] |= e2m1_encode(ldexpf(x[i], -ex)) << (4 * (i & 7));
    const int64_t e = slots ? slots[r] : r;
    *(uint4*)(codes + e * 64 + 16 * g) = make_uint4(w[0], w[1], w[2], w[3]);
    scales[e * 4 + g] = (uint8_t)(ex + 127);
}

// SWA (8-bit): e = floor(log2 amax) - 8; code = E4M3(x * 2^-e), saturating.
template <bool BF16>
__global__ __launch_bounds__(256) void pack_swa_kernel(const void* __restrict__ src, int64_t n,
                                                       int64_t stride, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales,
                                                       const int64_t* __restrict__ slots) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= n * 32) return;
    const int64_t r = gid >> 5;
    const int g = (int)(gid & 31);
    float x[16];
    load_group<BF16>(src, r * stride + 16 * g, 16, x);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
    const int ex = mx_exponent(amax, 8);
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i >> 2] |= e4m3_encode(ldexpf(x[i], -ex)) << (8 * (i & 3));
    const int64_t e = slots ? slots[r] : r;
    *(uint4*)(codes + e * 512 + 16 * g) = make_uint4(w[0], w[1], w[2], w[3]);
    scales[e * 32 + g] = (uint8_t)(ex + 127);
}

hipError_t launch_pack(int kind, const void* src, bool bf16, int64_t n, int64_t stride,
                       uint8_t* codes, uint8_t* scales, const int64_t* slots, hipStream_t st) {
    const int64_t groups = n * (kind == 1 ? 4 : 32);
    const dim3 grid((unsigned)((groups + 255) / 256)), block(256);
    if (kind == 0) {
        if (bf16) hipLaunchKernelGGL(pack_main_kernel<true>, grid, block, 0, st, src, n, stride, codes, scales, slots);
        else hipLaunchKernelGGL(pack_main_kernel<false>, grid, block, 0, st, src, n, stride, codes, scales, slots);
    } else if (kind == 1) {
        if (bf16) hipLaunchKernelGGL(pack_index_kernel<true>, grid, block, 0, st, src, n, stride, codes, scales, slots);
        else hipLaunchKernelGGL(pack_index_kernel<false>, grid, block, 0, st, src, n, stride, codes, scales, slots);
    } else {
        if (bf16) hipLaunchKernelGGL(pack_swa_kernel<true>, grid, block, 0, st, src, n, stride, codes, scales, slots);
        else hipLaunchKernelGGL(pack_swa_kernel<false>, grid, block, 0, st, src, n, stride, codes, scales, slots);
    }
    return hipGetLastError();
}

}  // namespace csa2
