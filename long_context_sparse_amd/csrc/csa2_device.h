// csa2_device.h -- device-side helpers shared by the CSA2 kernels (gfx950).
//
// Element codecs of the three storage formats (E2M1 / E4M3 / E8M0, from the
// OCP 8-bit floating point and Microscaling v1.0 format definitions), the
// KV-cache address map, and small wave-level utilities.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- KV view
struct KvView {
    const uint8_t* main_codes;
    const uint8_t* main_scales;
    const uint8_t* idx_codes;
    const uint8_t* idx_scales;
    const int32_t* page_table;
    int64_t req_stride;
    int32_t page_shift;   // log2(page_entries); -1 = contiguous
    int32_t max_pages;
};

// Entry id of position `pos` of request `req` (paged or contiguous layout).
__device__ __forceinline__ int64_t entry_of(const KvView& kv, int req, int pos) {
    if (kv.page_shift < 0) return (int64_t)req * kv.req_stride + pos;
    const int pg = pos >> kv.page_shift;
    const int off = pos & ((1 << kv.page_shift) - 1);
    return ((int64_t)kv.page_table[(int64_t)req * kv.max_pages + pg] << kv.page_shift) + off;
}

// ---------------------------------------------------------------- scalars
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
    const uint32_t b = __float_as_uint(x);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Value of an E2M1 code (bit 3 sign, bits 2:1 exponent with bias 1, bit 0
// mantissa; exponent 0 is subnormal 0.5*m), built as fp32 bits.
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
    const uint32_t m = c & 7u;
    uint32_t bits = (m >= 2u) ? ((((m >> 1) + 126u) << 23) | ((m & 1u) << 22))
                              : (m == 1u ? (126u << 23) : 0u);
    bits |= (c & 8u) << 28;
    return __uint_as_float(bits);
}

// Magnitude code of round-to-nearest-even onto {0,.5,1,1.5,2,3,4,6},
// saturating at 6: the number of decision points at or below a (each tie
// goes to the even mantissa).
__device__ __forceinline__ uint32_t e2m1_mag_code(float a) {
    return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
           (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
           (uint32_t)(a > 5.0f);
}

__device__ __forceinline__ uint32_t e2m1_encode(float y) {
    return e2m1_mag_code(fabsf(y)) | ((__float_as_uint(y) >> 28) & 8u);
}

// E4M3 (bias 7, no infinities, max 448) value of a code.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float v = (e == 0u) ? (float)m * 0.001953125f                       // m * 2^-9
                        : __uint_as_float(((e + 120u) << 23) | (m << 20));   // (1+m/8) 2^(e-7)
    return (c & 0x80u) ? -v : v;
}

// fp32 -> E4M3, round to nearest even on the mantissa bits, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
    const uint32_t b = __float_as_uint(x);
    const uint32_t sign = (b >> 24) & 0x80u;
    const float a = fabsf(x);
    if (!(a < 448.0f)) return sign | 0x7Eu;
    const uint32_t ab = b & 0x7FFFFFFFu;
    const int E = (int)(ab >> 23) - 127;
    if (E < -6) {                                   // E4M3 subnormal: step 2^-9
        const float q = rintf(a * 512.0f);
        return sign | (uint32_t)q;
    }
    const uint32_t mant = ab & 0x7FFFFFu;
    uint32_t keep = mant >> 20;
    const uint32_t rem = mant & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) keep++;
    uint32_t code = ((uint32_t)(E + 7) << 3) + keep;     // keep == 8 carries
    return sign | (code < 0x7Eu ? code : 0x7Eu);
}

// E8M0 exponent of an MX block: floor(log2 amax) - emax_elem, clamped to
// [-127, 127]; -127 for amax == 0 or an fp32-subnormal amax.
__device__ __forceinline__ int mx_exponent(float amax, int emax_elem) {
    const uint32_t f = __float_as_uint(amax) >> 23;
    int e = (f == 0u) ? -127 : (int)f - 127 - emax_elem;
    e = e < -127 ? -127 : e;
    return e > 127 ? 127 : e;
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
    // 2^(c-127): exponent field c for c >= 1; c == 0 is 2^-127 (fp32 subnormal)
    return (c == 0u) ? __uint_as_float(0x00400000u) : __uint_as_float(c << 23);
}

// ---------------------------------------------------------------- ordering
// Order-preserving map of finite floats to uint32 (larger float -> larger
// key); -0 is folded onto +0.  -inf maps to 0 = "absent"; every finite value
// maps to a key >= 0x00800000.
__device__ __forceinline__ uint32_t order_key(float f) {
    if (f == 0.0f) f = 0.0f;
    const uint32_t b = __float_as_uint(f);
    if (b == 0xFF800000u) return 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ---------------------------------------------------------------- waves
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// Max / sum of v over lanes l and l ^ 16 (or l ^ 32), without a trip through
// LDS: V_PERMLANE16_SWAP_B32 applied to two copies of v leaves rows (0, 0, 2,
// 2) of 16 lanes in one result and rows (1, 1, 3, 3) in the other
// (V_PERMLANE32_SWAP_B32: halves (0, 0) and (1, 1)), so combining the two
// combines every lane with its partner.  Both operations are commutative, so
// the result equals the shuffle-based form bit for bit.
__device__ __forceinline__ float max_xor16(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float add_xor16(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float shfl_up_f(float v, int d) { return __shfl_up(v, d, 64); }

}  // namespace csa2
