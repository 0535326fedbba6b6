// compress.hip -- the write path in front of the cache: compressed entries
// built from projected token streams, normalised, rotated and packed in one
// pass (gfx950).
//
// 'DeepSeek-V4' paper page:
//   * section 2.3.1: entry i of the overlapping compression is, per channel,
//     the softmax-weighted sum of the m value rows of block i (stream a) and
//     the m value rows of block i - 1 (stream b), the weights a softmax over
//     the 2m logits Z + B (positional bias per position in the block); entry
//     0 has no b part; the indexer keys take the same compression;
//   * section 2.3.2: the heavily compressed branch compresses blocks of m'
//     tokens without overlap;
//   * section 2.3.3: an RMSNorm of the compressed entry before attention and
//     a rotary embedding on its last 64 channels.
// 'KV cache diet' page: the entry is quantised after the rotation.
//
// MI355X mapping: one wave per entry.  Lane l holds `width / 64` consecutive
// channels (8 for the 512-channel latent, 2 for the 128-channel indexer key),
// so every token row is read as one contiguous, coalesced run per wave; the
// softmax over the block's rows is an online one in registers (running max,
// rescaled sum), the RMSNorm's sum of squares a wave reduction, and the
// quantisation groups (16 channels = 2 lanes, 32 channels = 16 lanes) are
// reduced with lane shuffles.  Rotation angles are formed and evaluated in
// fp64 (positions reach 2^20 and more, where an fp32 angle would be off by
// far more than the tolerance).  Quantisation uses the packer's rules and
// codecs, so the packed bytes are those csa2_pack_kv gives for the same
// values.  Memory-bound: 4m (or 2m') rows of `width` fp32 values read per
// entry, 288 or 68 bytes written.
#include <cmath>

#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

constexpr int CP_WAVES = 4;   // entries per workgroup

template <int CH>
__device__ __forceinline__ void load_ch(const float* p, float* x) {
    if constexpr (CH == 8) {
        const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
        const float2 a = *(const float2*)p;
        x[0] = a.x; x[1] = a.y;
    }
}

// Online softmax-weighted accumulation of `rows` token rows (logits z + b,
// values v) into (mx, s, acc), per channel.
// (values and logits: token rows of `stride` elements; biases: [rows][64 CH])
template <int CH>
__device__ __forceinline__ void accumulate(const float* v, const float* z, const float* b, int64_t t0, int rows,
                                           int64_t stride, int c0, float* mx, float* s, float* acc) {
    for (int k = 0; k < rows; ++k) {
        float vv[CH], zz[CH], bb[CH];
        load_ch<CH>(v + (t0 + k) * stride + c0, vv);
        load_ch<CH>(z + (t0 + k) * stride + c0, zz);
        load_ch<CH>(b + (int64_t)k * (64 * CH) + c0, bb);
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const float lg = zz[j] + bb[j];
            if (lg > mx[j]) {
                const float r = mx[j] == -INFINITY ? 0.0f : expf(mx[j] - lg);
                s[j] *= r;
                acc[j] *= r;
                mx[j] = lg;
            }
            const float p = expf(lg - mx[j]);
            s[j] += p;
            acc[j] = fmaf(p, vv[j], acc[j]);
        }
    }
}

// Blocks of M <= 4 tokens (M > 0): every row of the entry (M of stream a, M
// of stream b) is requested before any is used, then a two-pass softmax in
// registers.  M == 0: any block size, rows walked with an online softmax.
template <int WIDTH, int M>
__global__ __launch_bounds__(64 * CP_WAVES) void compress_pack_kernel(CompressArgs a, float* __restrict__ values,
                                                                     uint8_t* __restrict__ codes,
                                                                     uint8_t* __restrict__ scales,
                                                                     const int64_t* __restrict__ slots) {
    constexpr int CH = WIDTH / 64;
    const int64_t i = (int64_t)blockIdx.x * CP_WAVES + (threadIdx.x >> 6);
    if (i >= a.n_ent) return;                           // whole waves leave together
    const int l = threadIdx.x & 63;
    const int c0 = CH * l;
    float y[CH];
    if constexpr (M > 0) {
        const bool has_b = a.cb && i > 0;
        // rows 0..M-1: stream a of block i; rows M..2M-1: stream b of block i-1
        // (re-reading block i's a rows where there is no b part; masked below)
        float vv[2 * M][CH], zz[2 * M][CH], bs[2 * M][CH];
#pragma unroll
        for (int k = 0; k < M; ++k) {
            const int64_t ta = (i * M + k) * a.stride + c0;
            load_ch<CH>(a.ca + ta, vv[k]);
            load_ch<CH>(a.za + ta, zz[k]);
            load_ch<CH>(a.ba + k * WIDTH + c0, bs[k]);
            const int64_t tb = has_b ? ((i - 1) * M + k) * a.stride + c0 : ta;
            load_ch<CH>(has_b ? a.cb + tb : a.ca + tb, vv[M + k]);
            load_ch<CH>(has_b ? a.zb + tb : a.za + tb, zz[M + k]);
            load_ch<CH>((has_b ? a.bb : a.ba) + k * WIDTH + c0, bs[M + k]);
        }
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            float lg[2 * M];
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 2 * M; ++r) {
                lg[r] = (r < M || has_b) ? zz[r][j] + bs[r][j] : -INFINITY;
                mx = fmaxf(mx, lg[r]);
            }
            float sum = 0.0f, acc = 0.0f;
#pragma unroll
            for (int r = 0; r < 2 * M; ++r) {
                const float p = (r < M || has_b) ? expf(lg[r] - mx) : 0.0f;
                sum += p;
                acc = fmaf(p, vv[r][j], acc);
            }
            y[j] = acc / sum;
        }
    } else {
        float mx[CH], s[CH], acc[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j) { mx[j] = -INFINITY; s[j] = 0.0f; acc[j] = 0.0f; }
        // the entry's own block (stream a), then the block before it (stream b)
        accumulate<CH>(a.ca, a.za, a.ba, i * a.m, a.m, a.stride, c0, mx, s, acc);
        if (a.cb && i > 0) accumulate<CH>(a.cb, a.zb, a.bb, (i - 1) * a.m, a.m, a.stride, c0, mx, s, acc);
#pragma unroll
        for (int j = 0; j < CH; ++j) y[j] = acc[j] / s[j];
    }
    if (a.norm_weight) {
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < CH; ++j) ss = fmaf(y[j], y[j], ss);
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) ss += __shfl_xor(ss, d, 64);
        const float r = 1.0f / sqrtf(ss / (float)WIDTH + a.eps);
        float w[CH];
        load_ch<CH>(a.norm_weight + c0, w);
#pragma unroll
        for (int j = 0; j < CH; ++j) y[j] = y[j] * r * w[j];
    }
    if (a.rope && c0 >= WIDTH - 64) {
        // angle = pos * 10000^(-2j/64) in turns, formed in fp64 (exact to far
        // below an fp32 ulp of the reduced angle at any position < 2^40); its
        // integer turns removed there, the remaining fraction of a turn is an
        // fp32 angle in [-pi, pi] whose sine and cosine carry fp32 accuracy
        constexpr double INV_2PI = 0.15915494309189533577;
        const double pos = (double)(a.pos0 + i * a.m);
#pragma unroll
        for (int j = 0; j < CH; j += 2) {
            const int pair = (c0 + j - (WIDTH - 64)) >> 1;
            const double turns = pos * (a.inv_freq[pair] * INV_2PI);
            const float fr = (float)(turns - rint(turns));
            float sn, cs;
            sincosf(fr * 6.28318530717958647692f, &sn, &cs);
            const float x0 = y[j], x1 = y[j + 1];
            y[j] = fmaf(x0, cs, -x1 * sn);
            y[j + 1] = fmaf(x0, sn, x1 * cs);
        }
    }
    if (values) {
        float* vp = values + i * WIDTH + c0;
        if constexpr (CH == 8) {
            *(float4*)vp = make_float4(y[0], y[1], y[2], y[3]);
            *(float4*)(vp + 4) = make_float4(y[4], y[5], y[6], y[7]);
        } else {
            *(float2*)vp = make_float2(y[0], y[1]);
        }
    }
    const int64_t e = slots ? slots[i] : i;
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < CH; ++j) amax = fmaxf(amax, fabsf(y[j]));
    if constexpr (WIDTH == 512) {
        // MAIN: 16-channel groups = lanes (2g, 2g+1); s = E4M3(fl32(amax / 6))
        amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
        const uint32_t sc = e4m3_encode(__fdiv_rn(amax, 6.0f));
        const float sv = e4m3_to_f32(sc);
        uint32_t w = 0;
        if (sv != 0.0f) {
#pragma unroll
            for (int j = 0; j < 8; ++j) w |= e2m1_encode(__fdiv_rn(y[j], sv)) << (4 * j);
        }
        *(uint32_t*)(codes + e * 256 + 4 * l) = w;
        if ((l & 1) == 0) scales[e * 32 + (l >> 1)] = (uint8_t)sc;
    } else {
        // INDEX (MXFP4): 32-channel groups = 16 lanes; e = floor(log2 amax) - 2
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
        const int ex = mx_exponent(amax, 2);
        const uint32_t byte = e2m1_encode(ldexpf(y[0], -ex)) | (e2m1_encode(ldexpf(y[1], -ex)) << 4);
        codes[e * 64 + l] = (uint8_t)byte;
        if ((l & 15) == 0) scales[e * 4 + (l >> 4)] = (uint8_t)(ex + 127);
    }
}

hipError_t launch_compress_pack(const CompressArgs& a_in, int width, float* values, uint8_t* codes, uint8_t* scales,
                                const int64_t* slots, hipStream_t st) {
    CompressArgs a = a_in;
    for (int j = 0; j < 32; ++j) a.inv_freq[j] = std::pow(10000.0, -2.0 * j / 64.0);
    const dim3 grid((unsigned)((a.n_ent + CP_WAVES - 1) / CP_WAVES)), block(64 * CP_WAVES);
#define CP_LAUNCH(W, M) hipLaunchKernelGGL((compress_pack_kernel<W, M>), grid, block, 0, st, a, values, codes, scales, slots)
    const int m = a.m;   // the unrolled forms serve the overlapping compression of 1, 2 or 4 tokens
    const int mk = (a.cb && (m == 1 || m == 2 || m == 4)) ? m : 0;
    if (width == 512) {
        if (mk == 1) CP_LAUNCH(512, 1);
        else if (mk == 2) CP_LAUNCH(512, 2);
        else if (mk == 4) CP_LAUNCH(512, 4);
        else CP_LAUNCH(512, 0);
    } else {
        if (mk == 1) CP_LAUNCH(128, 1);
        else if (mk == 2) CP_LAUNCH(128, 2);
        else if (mk == 4) CP_LAUNCH(128, 4);
        else CP_LAUNCH(128, 0);
    }
#undef CP_LAUNCH
    return hipGetLastError();
}

}  // namespace csa2
