// attn.hip -- K4/K5: sparse attention over the selected FP4 entries, jointly
// with the 8-bit sliding window and an optional sink (gfx950).
//
// Shared-KV MQA: every selected compressed entry is both key and value, and
// the query heads attend in the 512-channel latent space (absorbed query)
// ['DeepSeek-V4' paper page, section 2.3.1 "Shared Key-Value MQA"; MLA article,
// section 4, matrix absorption].  The FP4 main entries are restored before
// attention [V4.1-Flash architecture page: FP4 storage is dequantised before
// the matmuls].  The sliding-window entries join the same softmax, and an
// optional per-head sink adds exp(z'_h) to the denominator [section 2.3.3].
//
// MI355X mapping
//   * A row's entries form one virtual list: its selected FP4 entries, padded
//     to a multiple of 64, then its window entries.  A workgroup walks a
//     contiguous range of 64-entry chunks with an online softmax, one wave per
//     16 heads.  Few rows (decode): each chunk gets its own workgroup and a
//     merge kernel combines the partials; many rows (prefill): one
//     workgroup per row writes the final output itself.
//   * Per chunk the workgroup gathers the 64 entries once and dequantises them
//     into LDS -- bf16 rows [entry][channel] for Q.K, and columns
//     [channel][entry] for P.V.  FP4 x E4M3 values have at most 6
//     significant bits and lie in [2^-10, 2688]: exact in bf16 and in fp16.
//     E2M1 codes become fp16 through a byte-permute table (V_PERM_B32), are
//     scaled with packed fp16 multiplies and turned into bf16 by exponent
//     re-biasing.  Window values E4M3 x 2^e are exact in bf16.
//   * Two waves per 16 heads: both compute the same scores, each does P.V for
//     half of the 512 channels (more waves in flight, half the accumulators).
//   * Split partials are stored normalised (O / l) in fp16 with (max, sum) in
//     fp32, which halves the merge traffic.
//   * S^T = K q^T on V_MFMA_F32_16X16X32_BF16 (A = 16 entries from LDS, B = the
//     wave's 16 query heads held in registers).  The MFMA output layout puts
//     4 consecutive entries of one head in a lane, which is exactly the
//     B-operand layout P^T needs for O^T = V^T P^T once the contraction slots
//     are mapped to entries {4g..4g+3, 16+4g..16+4g+3}: P never leaves
//     registers.  Selected chunks use V_MFMA_F32_16X16X32_F16 with P in fp16;
//     window chunks use bf16 with P split into a bf16 head and tail.
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int AT_ENT = 64;            // entries per chunk
constexpr int KT_LD = 512 + 8;        // bf16 elements per K row in LDS (padded)
constexpr int VT_LD = AT_ENT + 4;     // 16-bit elements per V^T row in LDS (padded)
constexpr size_t AT_LDS = (size_t)AT_ENT * KT_LD * 2 + (size_t)512 * VT_LD * 2;
constexpr int AT_MAX_SPLITS = 10;     // 512 selected + 128 window entries, 64 per chunk
constexpr int AT_HEADS_PER_WG = 64;

int attn_splits(int n_rows) {
    if (n_rows <= 0) return 1;
    const int s = (2560 + n_rows - 1) / n_rows;   // aim at ~2,560 workgroups
    return s < 1 ? 1 : (s > AT_MAX_SPLITS ? AT_MAX_SPLITS : s);
}

// per split and head: 512 fp16 (normalised partial output) + max + sum (fp32)
static size_t split_bytes(int n_heads) { return (size_t)n_heads * (512 * 2 + 8); }

size_t attn_workspace_bytes(int n_rows, int n_heads) {
    const int s = attn_splits(n_rows);
    if (s == 1) return 256;
    return (size_t)n_rows * s * split_bytes(n_heads);
}

// q B-operand of one wave: lane holds head (h0 + l%16), channels
// 32*ks + 8*(l/16) .. +8 for ks = 0..15, as bf16 (fp32 input rounded to nearest even).
template <bool QBF16>
__device__ __forceinline__ void load_q_operand(const void* q, int64_t row_head0, int n, int g, bf16x8* qv) {
    if (QBF16) {
        const uint16_t* p = (const uint16_t*)q + (row_head0 + n) * 512 + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) qv[ks] = *(const bf16x8*)(p + 32 * ks);
    } else {
        const float* p = (const float*)q + (row_head0 + n) * 512 + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            const float4 x0 = *(const float4*)(p + 32 * ks);
            const float4 x1 = *(const float4*)(p + 32 * ks + 4);
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            uint16_t b[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) b[i] = (uint16_t)f32_to_bf16_rne(xs[i]);
            qv[ks] = *(const bf16x8*)b;
        }
    }
}

// V^T A-operand for channel tile ct, contraction step u: channel 16ct + n,
// entries {32u + 4g .. +3} and {32u + 16 + 4g .. +3}.
__device__ __forceinline__ uint4 vt_operand(const uint16_t* Vt, int ct, int u, int n, int g) {
    const uint16_t* r = Vt + (16 * ct + n) * VT_LD + 32 * u + 4 * g;
    const uint2 lo = *(const uint2*)r;
    const uint2 hi = *(const uint2*)(r + 16);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// Eight E2M1 codes (one dword) -> four fp16 pairs (channels 2i, 2i+1).
// The fp16 high byte of each magnitude comes from a byte-permute table:
// 0, 0.5, 1, 1.5, 2, 3, 4, 6 = 0x00, 0x38, 0x3C, 0x3E, 0x40, 0x42, 0x44, 0x46.
__device__ __forceinline__ void e2m1x8_to_f16x2(uint32_t w, uint32_t* pr) {
    const uint32_t lut_lo = 0x3E3C3800u, lut_hi = 0x46444240u;
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    const uint32_t hb_lo = __builtin_amdgcn_perm(lut_hi, lut_lo, lo & 0x07070707u) | ((lo & 0x08080808u) << 4);
    const uint32_t hb_hi = __builtin_amdgcn_perm(lut_hi, lut_lo, hi & 0x07070707u) | ((hi & 0x08080808u) << 4);
    pr[0] = __builtin_amdgcn_perm(hb_hi, hb_lo, 0x040C000Cu);
    pr[1] = __builtin_amdgcn_perm(hb_hi, hb_lo, 0x050C010Cu);
    pr[2] = __builtin_amdgcn_perm(hb_hi, hb_lo, 0x060C020Cu);
    pr[3] = __builtin_amdgcn_perm(hb_hi, hb_lo, 0x070C030Cu);
}

// fp16 pair -> bf16 pair, exact for zero and for normal fp16 values whose
// mantissa fits in 7 bits (all dequantised FP4 x E4M3 values): re-bias the
// exponent by 127 - 15 = 112 and drop three zero mantissa bits.
__device__ __forceinline__ uint32_t f16x2_to_bf16x2_exact(uint32_t x) {
    const uint32_t t = x & 0x7FFF7FFFu, sgn = x & 0x80008000u;
    const uint32_t m = (t >> 3) & 0x0FFF0FFFu;
    const uint32_t nz = ((t + 0x7FFF7FFFu) >> 15) & 0x00010001u;   // per half: value != 0
    return sgn | (m + nz * 0x3800u);
}

__device__ __forceinline__ uint32_t pk_mul_f16(uint32_t a, uint32_t b) {
    const f16x2 r = __builtin_bit_cast(f16x2, a) * __builtin_bit_cast(f16x2, b);
    return __builtin_bit_cast(uint32_t, r);
}

// Gather + dequantise one chunk of selected FP4 entries (lane = entry); the
// loads of a lane's channel groups are all issued before any is used.
__device__ __forceinline__ void dequant_main_chunk(const KvView& kv, const AttnArgs& a, int row, int e0, int nent,
                                                   uint16_t* Kt, uint16_t* Vt, int wave, int W, int l) {
    const int j = l;
    const bool valid = j < nent;
    int64_t ent = 0;
    if (valid) ent = entry_of(kv, a.req[row], a.idx[(int64_t)row * a.idx_stride + e0 + j]);
    constexpr int GPW = 2;
    for (int g0 = wave; g0 < 32; g0 += W * GPW) {
        uint2 c[GPW];
        uint32_t sc[GPW];
#pragma unroll
        for (int k = 0; k < GPW; ++k) {
            const int grp = g0 + k * W;
            c[k] = make_uint2(0u, 0u);
            sc[k] = 0u;
            if (valid && grp < 32) {
                c[k] = *(const uint2*)(kv.main_codes + ent * 256 + 8 * grp);
                sc[k] = kv.main_scales[ent * 32 + grp];
            }
        }
#pragma unroll
        for (int k = 0; k < GPW; ++k) {
            const int grp = g0 + k * W;
            if (grp >= 32) break;
            const _Float16 sh = (_Float16)e4m3_to_f32(sc[k]);          // exact
            const uint32_t s2 = (uint32_t)__builtin_bit_cast(uint16_t, sh) * 0x00010001u;
            uint32_t hp[8], kb[8];
            e2m1x8_to_f16x2(c[k].x, hp);
            e2m1x8_to_f16x2(c[k].y, hp + 4);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                hp[i] = pk_mul_f16(hp[i], s2);                          // exact
                kb[i] = f16x2_to_bf16x2_exact(hp[i]);
                Vt[(16 * grp + 2 * i) * VT_LD + j] = (uint16_t)(hp[i] & 0xFFFFu);
                Vt[(16 * grp + 2 * i + 1) * VT_LD + j] = (uint16_t)(hp[i] >> 16);
            }
            uint4* kd = (uint4*)(Kt + j * KT_LD + 16 * grp);
            kd[0] = make_uint4(kb[0], kb[1], kb[2], kb[3]);
            kd[1] = make_uint4(kb[4], kb[5], kb[6], kb[7]);
        }
    }
}

// Load + dequantise one chunk of window entries (8-bit E4M3 x 2^e).
__device__ __forceinline__ void dequant_swa_chunk(const AttnArgs& a, int64_t first, int nent,
                                                  uint16_t* Kt, uint16_t* Vt, int wave, int W, int l) {
    const int j = l;
    const bool valid = j < nent;
    const int64_t ent = first + j;
    constexpr int GPW = 2;
    for (int g0 = wave; g0 < 32; g0 += W * GPW) {
        uint4 c[GPW];
        uint32_t sc[GPW];
#pragma unroll
        for (int k = 0; k < GPW; ++k) {
            const int grp = g0 + k * W;
            c[k] = make_uint4(0u, 0u, 0u, 0u);
            sc[k] = 127u;
            if (valid && grp < 32) {
                c[k] = *(const uint4*)(a.swa_codes + ent * 512 + 16 * grp);
                sc[k] = a.swa_scales[ent * 32 + grp];
            }
        }
#pragma unroll
        for (int k = 0; k < GPW; ++k) {
            const int grp = g0 + k * W;
            if (grp >= 32) break;
            const float s = e8m0_to_f32(sc[k]);
            const uint32_t words[4] = {c[k].x, c[k].y, c[k].z, c[k].w};
            uint32_t kb[8];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float v = e4m3_to_f32((words[i >> 2] >> (8 * (i & 3))) & 0xFFu) * s;
                const uint32_t bb = __float_as_uint(v) >> 16;          // exact bf16
                if (i & 1) kb[i >> 1] |= bb << 16; else kb[i >> 1] = bb;
                Vt[(16 * grp + i) * VT_LD + j] = (uint16_t)bb;
            }
            uint4* kd = (uint4*)(Kt + j * KT_LD + 16 * grp);
            kd[0] = make_uint4(kb[0], kb[1], kb[2], kb[3]);
            kd[1] = make_uint4(kb[4], kb[5], kb[6], kb[7]);
        }
    }
}

// Workgroup = (split, row, group of up to 64 heads); two waves per 16 heads
// (wave 2p and 2p+1 share heads 16p..16p+15 and take channel halves 0 / 1).
template <bool QBF16>
__global__ __launch_bounds__(512) void attn_kernel(KvView kv, AttnArgs a) {
    extern __shared__ __align__(16) uint8_t at_smem[];
    uint16_t* Kt = (uint16_t*)at_smem;
    uint16_t* Vt = Kt + AT_ENT * KT_LD;
    const int row = blockIdx.y, split = blockIdx.x;
    const int H = a.n_heads, W = blockDim.x >> 6;
    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int n = l & 15, g = l >> 4;
    const int half = wave & 1;
    const int h0 = blockIdx.z * AT_HEADS_PER_WG + (wave >> 1) * 16;
    const int nsp = a.idx ? min(a.idx_count[row], 512) : 0;
    const int nsw = a.swa_codes ? min(a.swa_count[row], 128) : 0;
    const int csp = (nsp + AT_ENT - 1) / AT_ENT;
    const int ctot = csp + (nsw + AT_ENT - 1) / AT_ENT;
    const int per = (ctot + a.n_splits - 1) / a.n_splits;
    const int cb = min(split * per, ctot), ce = min(cb + per, ctot);

    bf16x8 qv[16];
    load_q_operand<QBF16>(a.q, (int64_t)row * H + h0, n, g, qv);
    f32x4 oacc[16];
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) oacc[ct] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;

    for (int c = cb; c < ce; ++c) {
        const bool is_sw = c >= csp;
        const int e0 = is_sw ? (c - csp) * AT_ENT : c * AT_ENT;
        const int nent = min((is_sw ? nsw : nsp) - e0, AT_ENT);
        __syncthreads();                               // previous chunk fully consumed
        if (is_sw) dequant_swa_chunk(a, a.swa_first[row] + e0, nent, Kt, Vt, wave, W, l);
        else dequant_main_chunk(kv, a, row, e0, nent, Kt, Vt, wave, W, l);
        __syncthreads();
        // ---- S^T tiles: acc[et][i] = K[16et + 4g + i] . q[head n]
        f32x4 acc[4];
#pragma unroll
        for (int et = 0; et < 4; ++et) acc[et] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        {
            const uint16_t* base = Kt + n * KT_LD + 8 * g;
#pragma unroll
            for (int ks = 0; ks < 16; ++ks) {
#pragma unroll
                for (int et = 0; et < 4; ++et)
                    acc[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        *(const bf16x8*)(base + 16 * et * KT_LD + 32 * ks), qv[ks], acc[et], 0, 0, 0);
            }
        }
        // ---- online softmax (column = head)
        float m = -INFINITY;
#pragma unroll
        for (int et = 0; et < 4; ++et)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float z = (16 * et + 4 * g + i) < nent ? acc[et][i] * a.scale : -INFINITY;
                acc[et][i] = z;
                m = fmaxf(m, z);
            }
        m = fmaxf(m, shfl_xor_f(m, 16));
        m = fmaxf(m, shfl_xor_f(m, 32));
        const float m_new = fmaxf(m_run, m);
        const float alpha = (m_run == -INFINITY) ? 0.0f : expf(m_run - m_new);
        float lsum = 0.0f;
#pragma unroll
        for (int et = 0; et < 4; ++et)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = expf(acc[et][i] - m_new);
                acc[et][i] = p;
                lsum += p;
            }
        lsum += shfl_xor_f(lsum, 16);
        lsum += shfl_xor_f(lsum, 32);
        l_run = l_run * alpha + lsum;
        m_run = m_new;
        // ---- O^T += V^T P^T over this wave's 16 channel tiles
        const int ct0 = 16 * half;
        if (!is_sw) {
            f16x8 pb[2];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int i = 0; i < 8; ++i) pb[u][i] = (_Float16)acc[2 * u + (i >> 2)][i & 3];
#pragma unroll
            for (int ct = 0; ct < 16; ++ct) {
                f32x4 o = oacc[ct] * alpha;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const uint4 av = vt_operand(Vt, ct0 + ct, u, n, g);
                    o = __builtin_amdgcn_mfma_f32_16x16x32_f16(*(const f16x8*)&av, pb[u], o, 0, 0, 0);
                }
                oacc[ct] = o;
            }
        } else {
            bf16x8 phi[2], plo[2];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float p = acc[2 * u + (i >> 2)][i & 3];
                    const uint32_t hb = f32_to_bf16_rne(p);
                    const uint32_t lb = f32_to_bf16_rne(p - __uint_as_float(hb << 16));
                    phi[u][i] = __builtin_bit_cast(__bf16, (uint16_t)hb);
                    plo[u][i] = __builtin_bit_cast(__bf16, (uint16_t)lb);
                }
#pragma unroll
            for (int ct = 0; ct < 16; ++ct) {
                f32x4 o = oacc[ct] * alpha;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const uint4 av = vt_operand(Vt, ct0 + ct, u, n, g);
                    o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)&av, phi[u], o, 0, 0, 0);
                    o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)&av, plo[u], o, 0, 0, 0);
                }
                oacc[ct] = o;
            }
        }
    }

    const int h = h0 + n;
    const int cbase = 256 * half;                      // first channel of this wave
    if (a.n_splits > 1) {
        // normalised partial output (fp16) plus (max, sum) of this split
        const size_t ps = ((size_t)row * a.n_splits + split) * H + h;
        uint16_t* wsO = (uint16_t*)a.ws;
        float* wsM = (float*)(wsO + (size_t)a.n_rows * a.n_splits * H * 512);
        float* wsL = wsM + (size_t)a.n_rows * a.n_splits * H;
        if (cb < ce) {
            const float inv = 1.0f / l_run;
            uint16_t* orow = wsO + ps * 512 + cbase;
#pragma unroll
            for (int ct = 0; ct < 16; ++ct) {
                const _Float16 v0 = (_Float16)(oacc[ct][0] * inv), v1 = (_Float16)(oacc[ct][1] * inv);
                const _Float16 v2 = (_Float16)(oacc[ct][2] * inv), v3 = (_Float16)(oacc[ct][3] * inv);
                const uint2 pk = make_uint2((uint32_t)__builtin_bit_cast(uint16_t, v0) | ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16),
                                            (uint32_t)__builtin_bit_cast(uint16_t, v2) | ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16));
                *(uint2*)(orow + 16 * ct + 4 * g) = pk;
            }
        }
        if (g == 0 && half == 0) { wsM[ps] = m_run; wsL[ps] = l_run; }
        return;
    }
    // ---- single split: merge with the external partial and the sink here
    const float lse_p = a.lse_in ? a.lse_in[(int64_t)row * H + h] : -INFINITY;
    const float sk = a.sink ? a.sink[h] : -INFINITY;
    const float M = fmaxf(fmaxf(m_run, lse_p), sk);
    const float w_run = (m_run == -INFINITY) ? 0.0f : expf(m_run - M);
    const float w_p = (lse_p == -INFINITY) ? 0.0f : expf(lse_p - M);
    const float w_s = (sk == -INFINITY) ? 0.0f : expf(sk - M);
    const float den = w_run * l_run + w_p + w_s;
    const float inv = (M == -INFINITY || den == 0.0f) ? 0.0f : 1.0f / den;
    const float* oin = a.o_in ? a.o_in + ((int64_t)row * H + h) * 512 : nullptr;
    float* orow = a.out + ((int64_t)row * H + h) * 512;
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) {
        const int c = cbase + 16 * ct + 4 * g;
        const float4 pin = oin ? *(const float4*)(oin + c) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        float4 r;
        r.x = (w_run * oacc[ct][0] + w_p * pin.x) * inv;
        r.y = (w_run * oacc[ct][1] + w_p * pin.y) * inv;
        r.z = (w_run * oacc[ct][2] + w_p * pin.z) * inv;
        r.w = (w_run * oacc[ct][3] + w_p * pin.w) * inv;
        *(float4*)(orow + c) = r;
    }
    if (a.lse_out && g == 0 && half == 0)
        a.lse_out[(int64_t)row * H + h] = (M == -INFINITY || den == 0.0f) ? -INFINITY : M + logf(den);
}

// out = (sum_s e^(m_s - M) l_s o_s + e^(lse_in - M) o_in) / (sum_s e^(m_s - M) l_s + e^(lse_in - M) + e^(sink - M))
// with o_s the normalised fp16 partial of split s.  One thread per (head, 8 channels).
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
    const int H = a.n_heads, S = a.n_splits;
    const int row = blockIdx.y;
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= H * 64) return;
    const int h = t >> 6, c8 = t & 63;
    const uint16_t* wsO = (const uint16_t*)a.ws;
    const float* wsM = (const float*)(wsO + (size_t)a.n_rows * S * H * 512);
    const float* wsL = wsM + (size_t)a.n_rows * S * H;
    float ms[AT_MAX_SPLITS];
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) {
        ms[s] = wsM[((size_t)row * S + s) * H + h];
        M = fmaxf(M, ms[s]);
    }
    const float lse_p = a.lse_in ? a.lse_in[(int64_t)row * H + h] : -INFINITY;
    const float sk = a.sink ? a.sink[h] : -INFINITY;
    M = fmaxf(fmaxf(M, lse_p), sk);
    float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float den = 0.0f;
    if (M != -INFINITY) {
        for (int s = 0; s < S; ++s) {
            if (ms[s] == -INFINITY) continue;
            const size_t ps = ((size_t)row * S + s) * H + h;
            const float wgt = expf(ms[s] - M) * wsL[ps];
            den += wgt;
            const uint4 v = *(const uint4*)(wsO + ps * 512 + 8 * c8);
            const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f16x2 pr = __builtin_bit_cast(f16x2, wv[i]);
                o[2 * i] += wgt * (float)pr[0];
                o[2 * i + 1] += wgt * (float)pr[1];
            }
        }
        if (lse_p != -INFINITY) {
            const float wgt = expf(lse_p - M);
            den += wgt;
            const float* pin = a.o_in + ((int64_t)row * H + h) * 512 + 8 * c8;
            const float4 v0 = *(const float4*)pin, v1 = *(const float4*)(pin + 4);
            o[0] += wgt * v0.x; o[1] += wgt * v0.y; o[2] += wgt * v0.z; o[3] += wgt * v0.w;
            o[4] += wgt * v1.x; o[5] += wgt * v1.y; o[6] += wgt * v1.z; o[7] += wgt * v1.w;
        }
        if (sk != -INFINITY) den += expf(sk - M);
    }
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    float* orow = a.out + ((int64_t)row * H + h) * 512 + 8 * c8;
    *(float4*)orow = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
    *(float4*)(orow + 4) = make_float4(o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv);
    if (a.lse_out && c8 == 0) a.lse_out[(int64_t)row * H + h] = den > 0.0f ? M + logf(den) : -INFINITY;
}

static bool g_attr_set = false;

static hipError_t set_lds_attrs() {
    if (g_attr_set) return hipSuccess;
    hipError_t e;
    if ((e = hipFuncSetAttribute((const void*)attn_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)AT_LDS)) != hipSuccess) return e;
    if ((e = hipFuncSetAttribute((const void*)attn_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)AT_LDS)) != hipSuccess) return e;
    g_attr_set = true;
    return hipSuccess;
}

hipError_t launch_attn(const KvView& kv, const AttnArgs& a_in, hipStream_t st) {
    hipError_t e = set_lds_attrs();
    if (e != hipSuccess) return e;
    AttnArgs a = a_in;
    a.n_splits = attn_splits(a.n_rows);
    if (a.n_splits > a.max_chunks) a.n_splits = a.max_chunks > 0 ? a.max_chunks : 1;
    const int hg = (a.n_heads + AT_HEADS_PER_WG - 1) / AT_HEADS_PER_WG;
    const int heads_in_wg = a.n_heads < AT_HEADS_PER_WG ? a.n_heads : AT_HEADS_PER_WG;
    const dim3 grid((unsigned)a.n_splits, (unsigned)a.n_rows, (unsigned)hg);
    const dim3 block((unsigned)(2 * 64 * (heads_in_wg / 16)));
    if (a.q_bf16) hipLaunchKernelGGL(attn_kernel<true>, grid, block, AT_LDS, st, kv, a);
    else hipLaunchKernelGGL(attn_kernel<false>, grid, block, AT_LDS, st, kv, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.n_splits > 1) {
        const dim3 mgrid((unsigned)((a.n_heads * 64 + 255) / 256), (unsigned)a.n_rows);
        hipLaunchKernelGGL(attn_merge_kernel, mgrid, dim3(256), 0, st, a);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace csa2
