// index_score.hip -- K2: lightning-indexer scores over MXFP4 keys (gfx950).
//
// I_s = sum_h w_h * ReLU(q_h . K_s)  ['DeepSeek-V4' paper page, section 2.3.1,
// index-score equation], with the indexer attention in FP4 (section 2.3.4):
// the query heads are quantised to MXFP4 like the keys, each head's dot
// product is taken exactly and rounded once to fp32, and the heads are folded
// by a sequential fp32 fma chain from +0.
//
// Full scan: every visible position of the row, plus the max over each
// aligned group of 8 (the hierarchical indexer's block score, V4.1-Flash
// architecture page).  Pool mode: only the 8-position blocks of a given
// candidate pool (Reindex layers).
//
// Design (MI355X):
//   * HBM-bound stream of 68 B keys.  A wave takes 16 keys per step: lane l
//     loads 16 code bytes (key l%16, channel block l/16), so one wave load
//     covers 1 KB of contiguous codes; scales are one dword per key.
//   * The contraction runs on V_MFMA_SCALE_F32_16X16X128_F8F6F4 with both
//     operands in FP4 and E8M0 block scales: A = the row's indexer query
//     (heads on M, zero rows above n_heads), B = 16 keys (N).  K = 128 is
//     exactly the 4 MX blocks of a key.
//   * Exactness: every block term is S * 2^E with |S| <= 4608 quarter units
//     (13 bits).  If the exponents E of a head's 4 blocks span at most 9,
//     every partial sum is a multiple of 2^Emin below 2^(Emin+24), so fp32
//     accumulation in any order is exact and the MFMA result is the exactly
//     rounded value.  A per-key guard checks this (plus a range that keeps
//     every term a normal fp32); keys outside it are re-scored by an exact
//     integer path on the VALU.
//   * The fma fold follows the MFMA output layout: lanes 16g..16g+15 hold
//     heads 4g..4g+3 of the 16 keys; each lane group continues the chain
//     handed over by the previous one.
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

constexpr int IS_WAVES = 4;
constexpr int IS_TILES = 8;                          // 16-key tiles per wave
constexpr int IS_CHUNK = IS_WAVES * IS_TILES * 16;   // columns per workgroup

struct QShared {
    uint8_t codes[16][64];
    uint8_t scales[16][4];
    float w[16];
    int spread;   // max over real heads of (max - min) block scale code
    int smin;     // min block scale code over real heads
    int smax;     // max block scale code over real heads
};

// Doubled E2M1 value of a code, as an integer in {0, +-1, +-2, +-3, +-4, +-6, +-8, +-12}.
__device__ __forceinline__ int e2m1_x2(uint32_t nib) {
    const int m = (int)(nib & 7u);
    const int v = (m < 2) ? m : ((2 + (m & 1)) << ((m >> 1) - 1));
    return (nib & 8u) ? -v : v;
}

// Round-to-nearest-even fp32 of sum_t S[t] * 2^E[t] (4 terms, |S| < 2^20,
// -256 <= E <= 252), through a 576-bit two's-complement fixed point.
__device__ __noinline__ float round_pow2_sum4(const int* S, const int* E) {
    constexpr int NW = 9, OFF = 264;
    uint64_t L[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k) L[k] = 0;
    for (int t = 0; t < 4; ++t) {
        if (S[t] == 0) continue;
        const int p = E[t] + OFF;
        const int wd = p >> 6, b = p & 63;
        const int64_t v = S[t];
        const uint64_t lo = (uint64_t)v << b;
        const int64_t hi = (b == 0) ? (v >> 63) : (v >> (64 - b));
        const uint64_t ext = (v < 0) ? ~0ull : 0ull;
        uint64_t carry = 0;
        for (int k = wd; k < NW; ++k) {
            const uint64_t add = (k == wd) ? lo : ((k == wd + 1) ? (uint64_t)hi : ext);
            const uint64_t s1 = L[k] + add;
            const uint64_t c1 = s1 < add;
            const uint64_t s2 = s1 + carry;
            const uint64_t c2 = s2 < s1;
            L[k] = s2;
            carry = c1 | c2;
        }
    }
    const bool neg = (L[NW - 1] >> 63) != 0;
    if (neg) {
        uint64_t carry = 1;
        for (int k = 0; k < NW; ++k) {
            const uint64_t s = ~L[k] + carry;
            carry = (carry && s == 0) ? 1 : 0;
            L[k] = s;
        }
    }
    int top = -1;
    for (int k = NW - 1; k >= 0; --k)
        if (L[k]) { top = 64 * k + 63 - __clzll(L[k]); break; }
    if (top < 0) return 0.0f;
    int ulp = top - OFF - 23;
    if (ulp < -149) ulp = -149;
    const int cut = ulp + OFF;
    const int nb = top - cut + 1;                       // <= 24
    const int cw = cut >> 6, cb = cut & 63;
    uint64_t q = L[cw] >> cb;
    if (cb != 0 && cw + 1 < NW) q |= L[cw + 1] << (64 - cb);
    q &= (nb >= 64) ? ~0ull : ((1ull << nb) - 1);
    const int gpos = cut - 1;
    const int guard = (int)((L[gpos >> 6] >> (gpos & 63)) & 1ull);
    bool sticky = (L[gpos >> 6] & ((1ull << (gpos & 63)) - 1)) != 0;
    for (int k = 0; k < (gpos >> 6) && !sticky; ++k) sticky = L[k] != 0;
    if (guard && (sticky || (q & 1ull))) q++;
    const float r = ldexpf((float)q, ulp);
    return neg ? -r : r;
}

// Exact score of one key (used where the MFMA exactness guard fails).
__device__ __noinline__ float exact_key_score(const QShared& qs, int n_heads, const uint8_t* kc, const uint8_t* ks) {
    uint8_t key[64];
    for (int i = 0; i < 64; ++i) key[i] = kc[i];
    int kscale[4];
    for (int g = 0; g < 4; ++g) kscale[g] = ks[g];
    float acc = 0.0f;
    for (int h = 0; h < n_heads; ++h) {
        int S[4], E[4];
        for (int g = 0; g < 4; ++g) {
            int s = 0;
            for (int j = 0; j < 16; ++j) {
                const uint32_t qb = qs.codes[h][16 * g + j], kb = key[16 * g + j];
                s += e2m1_x2(qb & 15u) * e2m1_x2(kb & 15u) + e2m1_x2(qb >> 4) * e2m1_x2(kb >> 4);
            }
            S[g] = s;
            E[g] = (int)qs.scales[h][g] + kscale[g] - 256;
        }
        const float d = round_pow2_sum4(S, E);
        acc = fmaf(qs.w[h], d > 0.0f ? d : 0.0f, acc);
    }
    return acc == 0.0f ? 0.0f : acc;
}

// Quantise the row's indexer query to MXFP4 (one lane per (head, block) =
// exactly the MFMA A-operand layout) and gather the exactness-guard bounds.
template <bool QBF16>
__device__ void prep_query(QShared& qs, const void* q_idx, const float* w, int row, int n_heads) {
    const int l = threadIdx.x & 63;
    const int m = l & 15, g = l >> 4;
    uint32_t words[4] = {0, 0, 0, 0};
    int sc = 127;
    const bool real = m < n_heads;
    if (real) {
        float x[32];
        const int64_t off = ((int64_t)row * n_heads + m) * 128 + 32 * g;
        if (QBF16) {
            const uint16_t* p = (const uint16_t*)q_idx + off;
#pragma unroll
            for (int i = 0; i < 32; i += 8) {
                const uint4 v = *(const uint4*)(p + i);
                const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[i + 2 * j] = __uint_as_float(u[j] << 16);
                    x[i + 2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
                }
            }
        } else {
            const float* p = (const float*)q_idx + off;
#pragma unroll
            for (int i = 0; i < 32; ++i) x[i] = p[i];
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
        const int ex = mx_exponent(amax, 2);
#pragma unroll
        for (int i = 0; i < 32; ++i) words[i >> 3] |= e2m1_encode(ldexpf(x[i], -ex)) << (4 * (i & 7));
        sc = ex + 127;
    }
    *(uint4*)&qs.codes[m][16 * g] = make_uint4(words[0], words[1], words[2], words[3]);
    qs.scales[m][g] = (uint8_t)sc;
    if (l < 16) qs.w[l] = (l < n_heads) ? w[(int64_t)row * n_heads + l] : 0.0f;
    // per-head spread over its 4 blocks (lanes m, m+16, m+32, m+48)
    int mn = real ? sc : 1 << 20, mx = real ? sc : -(1 << 20);
    mn = min(mn, __shfl_xor(mn, 16, 64)); mx = max(mx, __shfl_xor(mx, 16, 64));
    mn = min(mn, __shfl_xor(mn, 32, 64)); mx = max(mx, __shfl_xor(mx, 32, 64));
    int spread = real ? mx - mn : 0;
    int smin = real ? mn : 1 << 20, smax = real ? mx : -(1 << 20);
    for (int d = 1; d < 16; d <<= 1) {
        spread = max(spread, __shfl_xor(spread, d, 64));
        smin = min(smin, __shfl_xor(smin, d, 64));
        smax = max(smax, __shfl_xor(smax, d, 64));
    }
    if (l == 0) { qs.spread = spread; qs.smin = smin; qs.smax = smax; }
}

template <bool QBF16, bool POOL>
__global__ __launch_bounds__(IS_WAVES * 64) void index_score_kernel(KvView kv, IndexScoreArgs a) {
    __shared__ QShared qs;
    const int row = blockIdx.y;
    const int nv = min(a.n_vis[row], a.max_vis);
    const int64_t pool_cap = a.pool_stride < 2048 ? a.pool_stride : 2048;
    const int ncols = POOL ? 8 * (int)min((int64_t)a.pool_count[row], pool_cap) : nv;
    const int chunk0 = blockIdx.x * IS_CHUNK;
    if (chunk0 >= ncols) return;                       // uniform over the workgroup
    const int req = a.req[row];
    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
    if (wave == 0) prep_query<QBF16>(qs, a.q_idx, a.w, row, a.n_heads);
    __syncthreads();

    const int n = l & 15, lg = l >> 4;
    const int NG = (a.n_heads + 3) >> 2;               // lane groups holding real heads
    i32x8 A = {0, 0, 0, 0, 0, 0, 0, 0};
    {
        const uint4 v = *(const uint4*)&qs.codes[n][16 * lg];
        A[0] = (int)v.x; A[1] = (int)v.y; A[2] = (int)v.z; A[3] = (int)v.w;
    }
    const int sa = qs.scales[n][lg];
    float wl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wl[i] = qs.w[min(4 * lg + i, 15)] * (4 * lg + i < a.n_heads ? 1.0f : 0.0f);
    const int qspread = qs.spread, qmin = qs.smin, qmax = qs.smax;
    const int32_t* pool = POOL ? a.pool + (int64_t)row * a.pool_stride : nullptr;
    float* srow = a.scores ? a.scores + (int64_t)row * a.scores_stride : nullptr;
    float* brow = (!POOL && a.block_max) ? a.block_max + (int64_t)row * a.block_max_stride : nullptr;
    const int nv8 = (nv + 7) & ~7;

    // ---- issue the loads of all tiles first
    uint4 kcode[IS_TILES];
    uint32_t kscl[IS_TILES];
    int kpos[IS_TILES];
    int64_t kent[IS_TILES];
#pragma unroll
    for (int t = 0; t < IS_TILES; ++t) {
        const int col0 = chunk0 + (wave * IS_TILES + t) * 16;
        const int col = col0 + n;
        const int c0 = col0 < ncols ? col0 : chunk0;
        int pos, ld;
        if (POOL) {
            const int cc = col < ncols ? col : c0;
            pos = col < ncols ? 8 * pool[col >> 3] + (col & 7) : 0x7FFFFFFF;
            ld = 8 * pool[cc >> 3] + (cc & 7);
            if (ld >= nv) ld = 8 * pool[cc >> 3];      // a visible position of the same block
        } else {
            pos = col;
            ld = col < nv ? col : c0;
        }
        kpos[t] = pos;
        const int64_t e = entry_of(kv, req, ld);
        kent[t] = e;
        kcode[t] = *(const uint4*)(kv.idx_codes + e * 64 + 16 * lg);
        kscl[t] = *(const uint32_t*)(kv.idx_scales + e * 4);
    }

    // ---- contraction, exactness guard, head fold, outputs
#pragma unroll
    for (int t = 0; t < IS_TILES; ++t) {
        const int col0 = chunk0 + (wave * IS_TILES + t) * 16;
        if (col0 >= ncols) break;
        i32x8 B = {(int)kcode[t].x, (int)kcode[t].y, (int)kcode[t].z, (int)kcode[t].w, 0, 0, 0, 0};
        const int sb = (int)((kscl[t] >> (8 * lg)) & 0xFFu);
        f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
        d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, d, 4, 4, 0, sa, 0, sb);

        const int b0 = kscl[t] & 0xFF, b1 = (kscl[t] >> 8) & 0xFF, b2 = (kscl[t] >> 16) & 0xFF, b3 = kscl[t] >> 24;
        const int kmin = min(min(b0, b1), min(b2, b3)), kmax = max(max(b0, b1), max(b2, b3));
        const bool ok = (kmax - kmin + qspread <= 9) && (qmin + kmin >= 136) && (qmax + kmax <= 356);

        float acc = 0.0f;
        for (int grp = 0; grp < NG; ++grp) {
            const float prev = shfl_up_f(acc, 16);
            float tt = grp == 0 ? 0.0f : prev;
#pragma unroll
            for (int i = 0; i < 4; ++i) tt = fmaf(wl[i], d[i] > 0.0f ? d[i] : 0.0f, tt);
            acc = (lg == grp) ? tt : acc;
        }
        acc = (acc == 0.0f) ? 0.0f : acc;
        const bool final_grp = (lg == NG - 1);
        if (__builtin_expect(__any(!ok), 0)) {
            if (final_grp && !ok)
                acc = exact_key_score(qs, a.n_heads, kv.idx_codes + kent[t] * 64, kv.idx_scales + kent[t] * 4);
        }
        const int col = col0 + n;
        const int pos = kpos[t];
        const bool vis = POOL ? (col < ncols && pos < nv) : (pos < nv);
        const float val = vis ? acc : -INFINITY;
        if (srow && final_grp) {
            if (POOL) { if (col < ncols) srow[col] = val; }
            else if (pos < nv8) srow[pos] = val;
        }
        if (!POOL && brow) {
            float bm = val;
            bm = fmaxf(bm, shfl_xor_f(bm, 1));
            bm = fmaxf(bm, shfl_xor_f(bm, 2));
            bm = fmaxf(bm, shfl_xor_f(bm, 4));
            if (final_grp && (n & 7) == 0 && pos < nv) brow[pos >> 3] = bm;
        }
    }
}

hipError_t launch_index_score(const KvView& kv, const IndexScoreArgs& a, hipStream_t st) {
    const bool pool = a.pool != nullptr;
    const int cols = pool ? 8 * 2048 : a.max_vis;
    const dim3 grid((unsigned)((cols + IS_CHUNK - 1) / IS_CHUNK), (unsigned)a.n_rows), block(IS_WAVES * 64);
    if (a.q_bf16) {
        if (pool) hipLaunchKernelGGL((index_score_kernel<true, true>), grid, block, 0, st, kv, a);
        else hipLaunchKernelGGL((index_score_kernel<true, false>), grid, block, 0, st, kv, a);
    } else {
        if (pool) hipLaunchKernelGGL((index_score_kernel<false, true>), grid, block, 0, st, kv, a);
        else hipLaunchKernelGGL((index_score_kernel<false, false>), grid, block, 0, st, kv, a);
    }
    return hipGetLastError();
}

}  // namespace csa2
