// synth.hip -- seeded synthetic inputs drawn on the GPU (counter-based).
//
// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014) used as a counter-based
// generator: base = mix64(seed * G + tensor), word(i) = mix64(base + (i+1) G).
// N(0,1) draws are the Irwin-Hall sum of twelve 16-bit fields of three words,
// centred and scaled by 2^-16, then rounded to bf16.  This lets very large
// caches be generated in place; the host generator of the test suite follows
// the same definition and the two are compared bit for bit.
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}

constexpr uint64_t GOLDEN = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t stream_word(uint64_t base, uint64_t i) { return mix64(base + (i + 1) * GOLDEN); }

__device__ __forceinline__ float irwin_hall(uint64_t base, uint64_t i) {
    int64_t tot = 0;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const uint64_t w = stream_word(base, 3 * i + k);
        tot += (int64_t)(w & 0xFFFF) + (int64_t)((w >> 16) & 0xFFFF) + (int64_t)((w >> 32) & 0xFFFF) +
               (int64_t)(w >> 48);
    }
    return (float)(tot - 393210) * (1.0f / 65536.0f);
}

template <bool BF16>
__global__ void synth_normal_kernel(uint64_t base, int64_t first, int64_t n, void* out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t b = f32_to_bf16_rne(irwin_hall(base, (uint64_t)(first + i)));
    if (BF16) ((uint16_t*)out)[i] = (uint16_t)b;
    else ((float*)out)[i] = __uint_as_float(b << 16);
}

__global__ void synth_uniform_kernel(uint64_t base, int64_t first, int64_t n, float* out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    out[i] = (float)(stream_word(base, (uint64_t)(first + i)) >> 40) * (1.0f / 16777216.0f);
}

__global__ void synth_boost_kernel(uint64_t base, int64_t first_pos, int64_t n_rows, int width, float* x) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_rows * width) return;
    const int64_t r = i / width;
    const uint64_t w = stream_word(base, (uint64_t)(first_pos + r));
    if (w < 922337203685477632ull) x[i] *= 3.0f;    // int(0.05 * 2^64)
}

static uint64_t host_mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}

static uint64_t stream_base(uint64_t seed, uint32_t tensor) { return host_mix64(seed * GOLDEN + tensor); }

hipError_t launch_synth_normal(uint64_t seed, uint32_t tensor, int64_t first, int64_t n, bool bf16, void* out,
                               hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const dim3 grid((unsigned)((n + 255) / 256)), block(256);
    if (bf16) hipLaunchKernelGGL(synth_normal_kernel<true>, grid, block, 0, st, stream_base(seed, tensor), first, n, out);
    else hipLaunchKernelGGL(synth_normal_kernel<false>, grid, block, 0, st, stream_base(seed, tensor), first, n, out);
    return hipGetLastError();
}

hipError_t launch_synth_uniform(uint64_t seed, uint32_t tensor, int64_t first, int64_t n, float* out,
                                hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(synth_uniform_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       stream_base(seed, tensor), first, n, out);
    return hipGetLastError();
}

hipError_t launch_synth_boost(uint64_t seed, uint32_t tensor, int64_t first_pos, int64_t n_rows, int width,
                              float* x, hipStream_t st) {
    const int64_t tot = n_rows * width;
    if (tot <= 0) return hipSuccess;
    hipLaunchKernelGGL(synth_boost_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st,
                       stream_base(seed, tensor), first_pos, n_rows, width, x);
    return hipGetLastError();
}

}  // namespace csa2
