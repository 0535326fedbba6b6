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
//     every term a normal fp32); the 8-blocks of keys outside it are queued in
//     LDS and re-scored after the main loop by an exact integer path.
//   * Each MFMA row group (rows 4g..4g+3) is given the same 4 query heads, so
//     every lane receives those 4 heads of its key; ceil(n_heads/4) MFMAs per
//     16 keys hand each lane all heads of its key, and the sequential fma fold
//     runs inside the lane with no cross-lane traffic (more than 16 heads: in
//     groups of 16, the fold continuing from group to group).  The block
//     maximum over 8 aligned keys uses DPP row shifts.
#include <algorithm>
#include <type_traits>

#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

#ifndef CSA2_IS_TILES
#define CSA2_IS_TILES 4
#endif
#ifndef CSA2_IS_ITERS
#define CSA2_IS_ITERS 4
#endif
constexpr int IS_WAVES = 4;
constexpr int IS_TILES = CSA2_IS_TILES;              // 16-key tiles per batch
constexpr int IS_ITERS = CSA2_IS_ITERS;              // batches per wave (even)
constexpr int IS_CHUNK = IS_WAVES * IS_TILES * 16 * IS_ITERS;   // columns of one slice of a workgroup
constexpr int IS_MAX_SLICES = 8;                     // slices of a row per workgroup, at most

// One row's indexer query in MXFP4, its weights and the exactness-guard bounds.
// A row's quantised indexer query for up to MH heads.
template <int MH>
struct QRowT {
    uint8_t codes[MH][64];
    uint8_t scales[MH][4];
    float w[MH];
    int spread;   // max over real heads of (max - min) block scale code
    int smin;     // min block scale code over real heads
    int smax;     // max block scale code over real heads
};
typedef QRowT<16> QRow;
constexpr int IS_MAX_HEADS = 64;                     // indexer heads of the single-row scan (16 per group)

template <int MH>
struct QShared {
    QRowT<MH> q;
    int st[4][3];  // more than 16 heads: each wave's (spread, min, max) over its group
    int n_fix;    // queued 8-blocks that need the exact path
    int fix[IS_MAX_SLICES * IS_CHUNK / 8];
    // pool mode: the pool entries of this workgroup's blocks (batch b of every
    // wave: slots 32 b .. 32 b + 31) and the row's entry 0 (slot IS_CHUNK / 8)
    int pool_l[IS_CHUNK / 8 + 1];
};

// Doubled E2M1 value of a code, as an integer in {0, +-1, +-2, +-3, +-4, +-6, +-8, +-12}.
__device__ __forceinline__ int e2m1_x2(uint32_t nib) {
    const int m = (int)(nib & 7u);
    const int v = (m < 2) ? m : ((2 + (m & 1)) << ((m >> 1) - 1));
    return (nib & 8u) ? -v : v;
}

// Round-to-nearest-even fp32 of sum_t S[t] * 2^E[t] (4 terms, |S| < 2^20,
// -256 <= E <= 252), through a 576-bit two's-complement fixed point.
__device__ float round_pow2_sum4(const int* S, const int* E) {
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

// Exact score of one key (used where the MFMA exactness guard fails) against
// one row's quantised query: codes [heads][64], scales [heads][4], weights.
__device__ float exact_key_score(const uint8_t (*qcodes)[64], const uint8_t (*qscales)[4], const float* qw,
                                 int n_heads, const uint8_t* kc, const uint8_t* ks) {
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
                const uint32_t qb = qcodes[h][16 * g + j], kb = key[16 * g + j];
                s += e2m1_x2(qb & 15u) * e2m1_x2(kb & 15u) + e2m1_x2(qb >> 4) * e2m1_x2(kb >> 4);
            }
            S[g] = s;
            E[g] = (int)qscales[h][g] + kscale[g] - 256;
        }
        const float d = round_pow2_sum4(S, E);
        acc = fmaf(qw[h], d > 0.0f ? d : 0.0f, acc);
    }
    return acc == 0.0f ? 0.0f : acc;
}

// The row's indexer query, raw: lane (head hoff + l%16, block g = l/16) holds
// the 32 channels it will quantise, as 16 bf16 pairs or 32 floats.
struct QRaw {
    uint32_t w[32];
};

// Lane (head hoff + l % 16, block l / 16).  Up to 8 heads (`halves`): lane
// (head l % 8, half (l / 8) % 2, block l / 16) holds the 16 channels of that
// half of the block, so every lane of the wave has work.
template <bool QBF16>
__device__ __forceinline__ void load_query(QRaw& r, const void* q_idx, int row, int n_heads, int hoff = 0,
                                           bool halves = false) {
    const int l = threadIdx.x & 63;
    const int m = hoff + (halves ? (l & 7) : (l & 15)), g = l >> 4;
    if (m >= n_heads) return;
    const int64_t off = ((int64_t)row * n_heads + m) * 128 + 32 * g + (halves ? 16 * ((l >> 3) & 1) : 0);
    const int nw = (QBF16 ? 4 : 8) >> (halves ? 1 : 0);     // 16-B loads
    if (QBF16) {
        const uint4* p = (const uint4*)((const uint16_t*)q_idx + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i >= nw) break;
            const uint4 v = p[i];
            r.w[4 * i] = v.x; r.w[4 * i + 1] = v.y; r.w[4 * i + 2] = v.z; r.w[4 * i + 3] = v.w;
        }
    } else {
        const uint4* p = (const uint4*)((const float*)q_idx + off);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i >= nw) break;
            const uint4 v = p[i];
            r.w[4 * i] = v.x; r.w[4 * i + 1] = v.y; r.w[4 * i + 2] = v.z; r.w[4 * i + 3] = v.w;
        }
    }
}

// Quantise heads hoff .. hoff+15 of the row's indexer query to MXFP4 (one
// lane per (head, block) = exactly the MFMA A-operand layout) and gather
// their exactness-guard bounds (spread, min, max; returned in every lane).
template <bool QBF16, class QR>
__device__ __forceinline__ void prep_query(QR& qs, const QRaw& r, const float* w, int row, int n_heads, int hoff,
                                           int& spread_out, int& smin_out, int& smax_out, bool halves = false) {
    const int l = threadIdx.x & 63;
    const int m = hoff + (halves ? (l & 7) : (l & 15)), g = l >> 4;
    uint32_t words[4] = {0, 0, 0, 0};
    int sc = 127;
    const bool real = m < n_heads;
    if (halves) {
        // 16 channels per lane; the block's scale needs the other half's
        // largest magnitude (lane l ^ 8)
        float x[16];
        if (QBF16) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                x[2 * j] = __uint_as_float(r.w[j] << 16);
                x[2 * j + 1] = __uint_as_float(r.w[j] & 0xFFFF0000u);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = __uint_as_float(r.w[i]);
        }
        float amax = 0.0f;
        if (real) {
#pragma unroll
            for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
        }
        amax = fmaxf(amax, __shfl_xor(amax, 8, 64));
        if (real) {
            const int ex = mx_exponent(amax, 2);
#pragma unroll
            for (int i = 0; i < 16; ++i) words[i >> 3] |= e2m1_encode(ldexpf(x[i], -ex)) << (4 * (i & 7));
            sc = ex + 127;
        }
        *(uint2*)&qs.codes[m][16 * g + 8 * ((l >> 3) & 1)] = make_uint2(words[0], words[1]);
        if (!(l & 8)) qs.scales[m][g] = (uint8_t)sc;
    } else {
        if (real) {
            float x[32];
            if (QBF16) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    x[2 * j] = __uint_as_float(r.w[j] << 16);
                    x[2 * j + 1] = __uint_as_float(r.w[j] & 0xFFFF0000u);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 32; ++i) x[i] = __uint_as_float(r.w[i]);
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
    }
    if (l < 16) qs.w[hoff + l] = (hoff + l < n_heads) ? w[(int64_t)row * n_heads + hoff + l] : 0.0f;
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
    spread_out = spread;
    smin_out = smin;
    smax_out = smax;
}

// Keys of one batch (IS_TILES tiles of 16) for one lane: 16 code bytes and the
// key's scale dword per tile.
struct KeyBatch {
    uint4 code[IS_TILES];
    uint32_t scl[IS_TILES];
};

template <bool POOL>
__device__ __forceinline__ int col_pos(const int32_t* pool, int col) {
    return POOL ? 8 * pool[col >> 3] + (col & 7) : col;
}

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// Issue the loads of one batch of this wave.  Columns past the end are
// clamped into range (the loads are always issued, so that the compiler can
// count outstanding loads exactly and never waits on a prefetched batch).
// Full scan: a 16-column tile lies inside one page, so its page-table entry
// is one wave-uniform load.
// Pool mode: the pool entry of a column comes from global memory (lpool NULL)
// or from the workgroup's LDS copy (slots lbase + block mod 32).
// PTE (paged full scan): tile t's page-table entry was loaded ahead into lane
// lbase + t of pte (see slice_pte).
template <bool POOL, bool PTE = false>
__device__ __forceinline__ void load_batch(const KvView& kv, int req, const int32_t* pool, const int* lpool, int lbase,
                                           int nv, int ncols, int col_base, int tstride, int n, int lg, KeyBatch& kb,
                                           int pte = 0) {
#pragma unroll
    for (int t = 0; t < IS_TILES; ++t) {
        const int col0 = col_base + tstride * t;         // wave-uniform
        int64_t e;
        if (POOL) {
            const int c0 = col0 < ncols ? col0 : 0;      // column 0 is always valid when ncols > 0
            const int col = col0 + n < ncols ? col0 + n : c0;
            const int pe = !lpool ? pool[col >> 3]
                                  : lpool[col0 < ncols ? lbase + ((col >> 3) & 31) : IS_CHUNK / 8];
            int ld = 8 * pe + (col & 7);
            if (ld >= nv) ld = 8 * pe;                   // a visible position of the same block
            e = entry_of(kv, req, ld);
        } else {
            const int t0 = col0 < ncols ? col0 : 0;
            const int off = min(n, ncols - 1 - t0);      // stays inside the tile
            int64_t base;
            if (kv.page_shift < 0) base = (int64_t)req * kv.req_stride + t0;
            else {
                const int pg = PTE ? __builtin_amdgcn_readlane(pte, lbase + t)
                                   : kv.page_table[(int64_t)req * kv.max_pages + (t0 >> kv.page_shift)];
                base = ((int64_t)pg << kv.page_shift) + (t0 & ((1 << kv.page_shift) - 1));
            }
            e = base + off;
        }
        // the key stream is read once per scan: non-temporal loads keep it from
        // displacing the score rows (read back right away by the selection)
        // in the caches, and measure about 7 % faster
        const u32x4v cv = __builtin_nontemporal_load((const u32x4v*)(kv.idx_codes + e * 64 + 16 * lg));
        kb.code[t] = make_uint4(cv.x, cv.y, cv.z, cv.w);
        kb.scl[t] = __builtin_nontemporal_load((const uint32_t*)(kv.idx_scales + e * 4));
    }
}

// max(x, +0) for finite x as one integer max on the bits: a negative float or
// -0 reads as a negative integer and becomes +0 (the float max would first
// quiet its operand, one more instruction per head and key).
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// max with the value of lane l - shift of the same 16-lane row (scores are
// never NaN, so the plain instruction is used without quieting its operands)
__device__ __forceinline__ float dpp_row_shr_max(float v, int shift) {
    int src = __builtin_bit_cast(int, v);
    int sh;
    switch (shift) {   // DPP control must be a constant
        case 1: sh = __builtin_amdgcn_update_dpp(src, src, 0x111, 0xF, 0xF, false); break;
        case 2: sh = __builtin_amdgcn_update_dpp(src, src, 0x112, 0xF, 0xF, false); break;
        default: sh = __builtin_amdgcn_update_dpp(src, src, 0x114, 0xF, 0xF, false); break;
    }
    float r;
    asm volatile("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(v), "v"(__builtin_bit_cast(float, sh)));
    return r;
}

// Paged full scan: the page-table entries of the IS_ITERS x IS_TILES tiles of
// a wave's slice, tile t of batch b in lane 4 b + t (lanes 16 .. 63 repeat
// them), loaded one slice ahead so that no key load waits for one.  Columns
// past ncols use page 0, as load_batch does.
__device__ __forceinline__ int slice_pte(const KvView& kv, int req, int ncols, int sbase, int bstride, int tstride,
                                         int l) {
    static_assert(IS_ITERS * IS_TILES <= 64, "one lane per tile of a slice");
    if (kv.page_shift < 0) return 0;
    const int j = l % (IS_ITERS * IS_TILES);
    const int col0 = sbase + (j / IS_TILES) * bstride + tstride * (j % IS_TILES);
    const int t0 = col0 < ncols ? col0 : 0;
    return kv.page_table[(int64_t)req * kv.max_pages + (t0 >> kv.page_shift)];
}

// MULTI: a full scan whose workgroups take more than one slice of their row;
// PTE: a full scan of a paged cache (page-table entries loaded ahead).
// NM = ceil(heads / 4) MFMAs per tile for up to 16 heads, each giving all
// lanes the same 4 heads; NM = 0: more than 16 heads, one MFMA per group of
// 16 heads and tile, transposed over the lanes before the fold.  The query
// operands stay in registers for the whole scan.
template <bool QBF16, bool POOL, int NM, bool MULTI, bool PTE>
__device__ __forceinline__ void index_score_body(const KvView& kv, const IndexScoreArgs& a) {
    constexpr bool GROUPED = NM == 0;
    constexpr int NMR = GROUPED ? 4 : NM;             // MFMAs per head group
    __shared__ __align__(16) QShared<GROUPED ? IS_MAX_HEADS : 16> qs;
    const int row = blockIdx.y;
    const int nv = min(a.n_vis[row], a.max_vis);
    const int64_t pool_cap = a.pool_stride < 2048 ? a.pool_stride : 2048;
    const int ncols = POOL ? 8 * (int)min((int64_t)a.pool_count[row], pool_cap) : nv;
    // A wave takes batches of IS_TILES consecutive 16-column tiles (64 keys,
    // 4 KB of codes); batch b of wave w of workgroup x starts at column
    // 64 ((b Gx + x) IS_WAVES + w), so the resident waves of a row read one
    // compact run of consecutive batches.
    const int Gx = gridDim.x;
    static_assert(IS_TILES == 4, "a batch is one tile per lane group");
    static_assert(8 * IS_WAVES == 32 && IS_CHUNK / 8 <= IS_WAVES * 64, "a batch spans 32 blocks of the LDS pool copy");
    if (64 * IS_WAVES * (int)blockIdx.x >= ncols) return;   // uniform over the workgroup
    const int req = a.req[row];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
    const int n = l & 15, lg = l >> 4;
    const int32_t* pool = POOL ? a.pool + (int64_t)row * a.pool_stride : nullptr;
    const int wbase = 64 * (IS_WAVES * (int)blockIdx.x + wave);   // first column of this wave's first batch
    constexpr int TSTRIDE = 16;                        // columns between the tiles of a batch
    const int BSTRIDE = 64 * IS_WAVES * Gx;            // columns between a wave's batches

    QRaw qraw;
    const int ng = GROUPED ? (a.n_heads + 15) >> 4 : 1;   // head groups of 16; wave w prepares group w
    // up to 8 heads: every lane of wave 0 quantises half a block (the other
    // waves wait for it at the barrier below)
    const bool halves = !GROUPED && a.n_heads <= 8;
    if (wave < ng) load_query<QBF16>(qraw, a.q_idx, row, a.n_heads, 16 * wave, halves);   // issued before the keys
    KeyBatch A, B;
    int pte = PTE && !POOL ? slice_pte(kv, req, ncols, wbase, BSTRIDE, TSTRIDE, l) : 0;
    load_batch<POOL, PTE && !POOL>(kv, req, pool, nullptr, 0, nv, ncols, wbase, TSTRIDE, n, lg, A, pte);   // in flight during the query prep
    if (POOL && (int)threadIdx.x <= IS_CHUNK / 8) {
        // batch b's blocks of every wave: 32 (IS_WAVES x + Gx IS_WAVES b) / 4 + 0 .. 31
        const int t = threadIdx.x;
        const int gi = t == IS_CHUNK / 8 ? 0 : 8 * IS_WAVES * ((int)blockIdx.x + Gx * (t >> 5)) + (t & 31);
        qs.pool_l[t] = gi < (ncols >> 3) ? pool[gi] : 0;
    }
    if (wave < ng) {
        int sp, mn, mx;
        prep_query<QBF16>(qs.q, qraw, a.w, row, a.n_heads, 16 * wave, sp, mn, mx, halves);
        if (l == 0) {
            if (GROUPED) { qs.st[wave][0] = sp; qs.st[wave][1] = mn; qs.st[wave][2] = mx; }
            else { qs.q.spread = sp; qs.q.smin = mn; qs.q.smax = mx; }
        }
    }
    if (threadIdx.x == 0) qs.n_fix = 0;
    __syncthreads();

    // Up to 16 heads: MFMA k takes heads 4k .. 4k+3 on every row group (row n
    // carries head 4k + (n & 3)).  More than 16 heads: MFMA g takes the 16
    // heads of group g, one per row (row n carries head 16g + n).
    // (the transposed layout measured slower than this one for 8 heads, where
    // the scan is bound by HBM: it serves more than 16 heads only)
    constexpr bool TRANS = GROUPED;
    constexpr int NA = GROUPED ? IS_MAX_HEADS / 16 : NMR;
    constexpr int NS = 4;                              // row groups of 4 heads folded per head group
    i32x8 Aq[NA];
    int sa[NA];
    float wl[TRANS ? 1 : 4 * NMR];
#pragma unroll
    for (int k = 0; k < NA; ++k) {
        const int h = TRANS ? 16 * k + n : 4 * k + (n & 3);
        const uint4 v = *(const uint4*)&qs.q.codes[h][16 * lg];   // group rows above ng: unused
        Aq[k] = (i32x8){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        sa[k] = qs.q.scales[h][lg];
        if (!TRANS) {
#pragma unroll
            for (int i = 0; i < 4; ++i) wl[4 * k + i] = qs.q.w[4 * k + i];   // 0 above n_heads
        }
    }
    int qspread, qmin, qmax;
    if (GROUPED) {
        qspread = 0; qmin = 1 << 20; qmax = -(1 << 20);
        for (int g = 0; g < ng; ++g) {
            qspread = max(qspread, qs.st[g][0]); qmin = min(qmin, qs.st[g][1]); qmax = max(qmax, qs.st[g][2]);
        }
    } else {
        qspread = qs.q.spread; qmin = qs.q.smin; qmax = qs.q.smax;
    }
    float* srow = a.scores ? a.scores + (int64_t)row * a.scores_stride : nullptr;
    float* brow = (!POOL && a.block_max) ? a.block_max + (int64_t)row * a.block_max_stride : nullptr;
    const int nv8 = (nv + 7) & ~7;
    const bool writer = lg == 0;                       // up to 16 heads: the 4 row groups hold identical results

    // One batch: tile t's MFMAs leave key 16t + n's score in every lane n of
    // each row group; lane l keeps the one of tile l / 16, so the batch's 64
    // scores leave in one coalesced 256-B store, and its 8 block maxima in one
    // 32-B store.
    //
    // More than 16 heads: MFMA (g, t) leaves heads 16g + 4 lg + i (i = 0..3)
    // of key 16t + n in lane (n, lg).  A 4 x 4 transpose of (tile, row group)
    // over the lanes -- V_PERMLANE32_SWAP_B32 between tiles t and t + 2, then
    // V_PERMLANE16_SWAP_B32 between tiles t and t + 1 -- hands lane (n, lg)
    // all 16 heads of group g for key 16 lg + n, the key whose score it stores,
    // so each lane folds its own key's heads in head order and no MFMA or fma
    // is repeated.
    auto compute_grouped = [&](const KeyBatch& kb, int col_base, int lbase) __attribute__((always_inline)) {
        float acc = 0.0f;
#pragma unroll
        for (int g = 0; g < NA; ++g) {
            if (g >= ng) break;                        // uniform
            f32x4 d[IS_TILES];
#pragma unroll
            for (int t = 0; t < IS_TILES; ++t) {
                const i32x8 Bk = {(int)kb.code[t].x, (int)kb.code[t].y, (int)kb.code[t].z, (int)kb.code[t].w, 0, 0, 0, 0};
                const int sb = (int)((kb.scl[t] >> (8 * lg)) & 0xFFu);
                const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
                d[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Aq[g], Bk, z, 4, 4, 0, sa[g], 0, sb);
            }
            // pinned in wave-uniform control flow, as below
#pragma unroll
            for (int t = 0; t < IS_TILES; ++t) asm volatile("" : "+v"(d[t]));
            float hv[4][4];                            // [source row group s][i]: head 16g + 4s + i
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const auto p02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(d[0][i]), __float_as_uint(d[2][i]), false, false);
                const auto p13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(d[1][i]), __float_as_uint(d[3][i]), false, false);
                const auto q01 = __builtin_amdgcn_permlane16_swap(p02[0], p13[0], false, false);
                hv[0][i] = __uint_as_float(q01[0]);
                hv[1][i] = __uint_as_float(q01[1]);
                if (NS > 2) {
                    const auto q23 = __builtin_amdgcn_permlane16_swap(p02[1], p13[1], false, false);
                    hv[2][i] = __uint_as_float(q23[0]);
                    hv[3][i] = __uint_as_float(q23[1]);
                }
            }
            const float4* wg = (const float4*)&qs.q.w[16 * g];   // 0 above n_heads
#pragma unroll
            for (int s4 = 0; s4 < NS; ++s4) {
                const float4 w4 = wg[s4];
                acc = fmaf(w4.x, relu_bits(hv[s4][0]), acc);
                acc = fmaf(w4.y, relu_bits(hv[s4][1]), acc);
                acc = fmaf(w4.z, relu_bits(hv[s4][2]), acc);
                acc = fmaf(w4.w, relu_bits(hv[s4][3]), acc);
            }
        }
        const uint32_t sd = lg == 0 ? kb.scl[0] : (lg == 1 ? kb.scl[1] : (lg == 2 ? kb.scl[2] : kb.scl[3]));
        const int b0 = sd & 0xFF, b1 = (sd >> 8) & 0xFF, b2 = (sd >> 16) & 0xFF, b3 = sd >> 24;
        const int kmin = min(min(b0, b1), min(b2, b3)), kmax = max(max(b0, b1), max(b2, b3));
        const bool ok = (kmax - kmin + qspread <= 9) && (qmin + kmin >= 136) && (qmax + kmax <= 356);
        acc = (acc == 0.0f) ? 0.0f : acc;
        const int col = col_base + l;                  // = col_base + 16 lg + n
        const bool in_cols = col < ncols;
        const int pos = POOL ? (in_cols ? 8 * qs.pool_l[lbase + ((col >> 3) & 31)] + (col & 7) : 0x7FFFFFFF) : col;
        if (__builtin_expect(__any(!ok), 0)) {
            int bad = (!ok && in_cols && pos < nv) ? 1 : 0;
            bad |= __builtin_amdgcn_update_dpp(0, bad, 0x111, 0xF, 0xF, false);   // row_shr:1
            bad |= __builtin_amdgcn_update_dpp(0, bad, 0x112, 0xF, 0xF, false);   // row_shr:2
            bad |= __builtin_amdgcn_update_dpp(0, bad, 0x114, 0xF, 0xF, false);   // row_shr:4
            if ((n & 7) == 7 && bad) qs.fix[atomicAdd(&qs.n_fix, 1)] = col & ~7;
        }
        return (in_cols && pos < nv) ? acc : -INFINITY;
    };

    auto compute = [&](const KeyBatch& kb, int col_base, int lbase) __attribute__((always_inline)) {
        float val;
        if constexpr (TRANS) {
            val = compute_grouped(kb, col_base, lbase);
        } else {
        float vt[IS_TILES];
#pragma unroll
        for (int t = 0; t < IS_TILES; ++t) {
            vt[t] = -INFINITY;
            const int col0 = col_base + TSTRIDE * t;
            if (col0 >= ncols) break;
            const i32x8 Bk = {(int)kb.code[t].x, (int)kb.code[t].y, (int)kb.code[t].z, (int)kb.code[t].w, 0, 0, 0, 0};
            const uint32_t sd = kb.scl[t];
            const int sb = (int)((sd >> (8 * lg)) & 0xFFu);
            float acc = 0.0f;
            {
                f32x4 d[NMR];
#pragma unroll
                for (int k = 0; k < NMR; ++k) {
                    const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
                    d[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Aq[k], Bk, z, 4, 4, 0, sa[k], 0, sb);
                }
                // An MFMA takes operands from all 64 lanes: an opaque use pins it in
                // wave-uniform control flow (the compiler may otherwise sink it into
                // a lane-masked branch, where it returns wrong sums).
#pragma unroll
                for (int k = 0; k < NMR; ++k) asm volatile("" : "+a"(d[k]));
#pragma unroll
                for (int k = 0; k < NMR; ++k)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc = fmaf(wl[4 * k + i], relu_bits(d[k][i]), acc);
            }
            const int b0 = sd & 0xFF, b1 = (sd >> 8) & 0xFF, b2 = (sd >> 16) & 0xFF, b3 = sd >> 24;
            const int kmin = min(min(b0, b1), min(b2, b3)), kmax = max(max(b0, b1), max(b2, b3));
            const bool ok = (kmax - kmin + qspread <= 9) && (qmin + kmin >= 136) && (qmax + kmax <= 356);
            acc = (acc == 0.0f) ? 0.0f : acc;
            const int col = col0 + n;
            const bool in_cols = col < ncols;
            // full scan: the position is the column (padding up to a multiple of 8 gets -inf)
            const int pos = POOL ? (in_cols ? 8 * qs.pool_l[lbase + ((col >> 3) & 31)] + (col & 7) : 0x7FFFFFFF) : col;
            // an 8-block with an unguarded visible key is queued once (lanes 8j + 7)
            if (__builtin_expect(__any(!ok), 0)) {
                int bad = (!ok && in_cols && pos < nv) ? 1 : 0;
                bad |= __builtin_amdgcn_update_dpp(0, bad, 0x111, 0xF, 0xF, false);   // row_shr:1
                bad |= __builtin_amdgcn_update_dpp(0, bad, 0x112, 0xF, 0xF, false);   // row_shr:2
                bad |= __builtin_amdgcn_update_dpp(0, bad, 0x114, 0xF, 0xF, false);   // row_shr:4
                if (writer && (n & 7) == 7 && bad) qs.fix[atomicAdd(&qs.n_fix, 1)] = col & ~7;
            }
            vt[t] = (in_cols && pos < nv) ? acc : -INFINITY;
        }
        val = lg == 0 ? vt[0] : (lg == 1 ? vt[1] : (lg == 2 ? vt[2] : vt[3]));
        }
        const int col = col_base + l;                  // = col_base + 16 lg + n
        const bool in_cols = col < ncols;
        if (srow) {
            if (POOL) { if (in_cols) srow[col] = val; }
            else if (col < nv8) srow[col] = val;
        }
        if (!POOL && brow) {
            float bm = dpp_row_shr_max(val, 1);
            bm = dpp_row_shr_max(bm, 2);
            bm = dpp_row_shr_max(bm, 4);
            // lanes 8j + 7 now hold the maximum of keys 8j .. 8j+7 of the batch
            if ((n & 7) == 7 && (col & ~7) < nv) brow[col >> 3] = bm;
        }
    };

    // One slice: IS_ITERS batches per wave, the next batch always in flight;
    // MORE also fetches the first batch of the next slice.
    // lbase: pool mode, the batch's slots in the LDS pool copy; paged full
    // scan, its tiles' lanes in pte (pte_next: those of the next slice)
    auto slice = [&](auto more, const int sbase, const int pte_next) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < IS_ITERS; b += 2) {
            const int c_a = sbase + b * BSTRIDE, c_b = c_a + BSTRIDE;
            load_batch<POOL, PTE && !POOL>(kv, req, pool, qs.pool_l, POOL ? 32 * (b + 1) : IS_TILES * (b + 1), nv, ncols, c_b,
                                    TSTRIDE, n, lg, B, pte);
            compute(A, c_a, 32 * b);
            const int c_n = c_b + BSTRIDE;
            if (b + 2 < IS_ITERS || decltype(more)::value)
                load_batch<POOL, PTE && !POOL>(kv, req, pool, qs.pool_l,
                                        POOL ? 32 * ((b + 2) % IS_ITERS) : IS_TILES * ((b + 2) % IS_ITERS), nv, ncols,
                                        c_n, TSTRIDE, n, lg, A, b + 2 < IS_ITERS ? pte : pte_next);
            compute(B, c_b, 32 * (b + 1));
        }
    };
    // slices s = 0 .. nsl-1 of this workgroup start SSTRIDE columns apart
    // (pool mode: one slice covers the largest pool; without MULTI the grid
    // gives every slice its own workgroup)
    const int SSTRIDE = IS_ITERS * BSTRIDE;
    const int nsl = MULTI && !POOL ? (ncols - 64 * IS_WAVES * (int)blockIdx.x + SSTRIDE - 1) / SSTRIDE : 1;
    for (int s = 0; s + 1 < nsl; ++s) {
        const int pn = PTE ? slice_pte(kv, req, ncols, wbase + (s + 1) * SSTRIDE, BSTRIDE, TSTRIDE, l) : 0;
        slice(std::true_type(), wbase + s * SSTRIDE, pn);
        pte = pn;
    }
    slice(std::false_type(), wbase + (nsl - 1) * SSTRIDE, pte);

    // ---- exact path for the queued 8-blocks (first column of each)
    __syncthreads();
    const int nfix = qs.n_fix;
    for (int i = threadIdx.x; i < nfix; i += blockDim.x) {
        const int c8 = qs.fix[i];
        float bm = -INFINITY;
        for (int j = 0; j < 8; ++j) {
            const int col = c8 + j;
            if (col >= ncols) break;
            const int pos = col_pos<POOL>(pool, col);
            float v = -INFINITY;
            if (pos < nv) {
                const int64_t e = entry_of(kv, req, pos);
                v = exact_key_score(qs.q.codes, qs.q.scales, qs.q.w, a.n_heads, kv.idx_codes + e * 64, kv.idx_scales + e * 4);
            }
            if (srow) srow[col] = v;                   // col == pos in a full scan
            bm = fmaxf(bm, v);
        }
        if (brow) brow[c8 >> 3] = bm;
    }
}

template <bool QBF16, bool POOL, int NM, bool MULTI, bool PTE>
__global__ __launch_bounds__(IS_WAVES * 64) void index_score_kernel(KvView kv, IndexScoreArgs a) {
    index_score_body<QBF16, POOL, NM, MULTI, PTE>(kv, a);
}

// More than 16 heads.  The declared floor of 2 waves per SIMD caps the
// kernel at 256 registers, so the compiler gives the MFMAs VGPR results (the
// transpose reads them right away) instead of AGPRs copied out one by one.
template <bool QBF16, bool POOL, bool MULTI, bool PTE>
__global__ __launch_bounds__(IS_WAVES * 64) __attribute__((amdgpu_waves_per_eu(2))) void index_score_heads_kernel(
    KvView kv, IndexScoreArgs a) {
    index_score_body<QBF16, POOL, 0, MULTI, PTE>(kv, a);
}

// ---------------------------------------------------------------- rows of one request
// Chunked prefill: the query rows of one request score the same keys.  A
// workgroup takes RG groups of 4 rows and the columns of SR_ITERS batches per
// wave; every 16-key tile is loaded once and scored against all of its rows.
// MFMA k of row group rg carries row 4 rg + n/4, head 4k + n%4 on its M row n,
// so lane (n, lg) receives heads 4k .. 4k+3 of (row 4 rg + lg, key n) and
// folds them in the same order as the single-row kernel: the scores are the
// same bits.  Rows past the end of the call and columns past a row's visible
// count are computed but never stored.
constexpr int SR_ITERS = 16;                           // batches per wave (even)
constexpr int SR_CHUNK = IS_WAVES * IS_TILES * 16 * SR_ITERS;

template <int RG>
struct SharedRowsLds {
    QRow q[4 * RG];
    int n_fix;
    int fix_col[4 * RG * SR_CHUNK / 8];               // first column of a queued (row, 8-block)
    uint8_t fix_row[4 * RG * SR_CHUNK / 8];           // its row within the workgroup
};

// The declared floor of 2 waves per SIMD (the kernel's register count gives
// 2 anyway) lets the compiler put the MFMA results in VGPRs.
template <bool QBF16, int NM, int RG>
__global__ __launch_bounds__(IS_WAVES * 64) __attribute__((amdgpu_waves_per_eu(2))) void index_score_shared_kernel(
    KvView kv, IndexScoreArgs a, int req) {
    constexpr int R = 4 * RG;
    __shared__ SharedRowsLds<RG> sh;
    const int r0 = (int)blockIdx.y * R;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
    const int n = l & 15, lg = l >> 4;
    // visible counts of the lane's rows (4 rg + lg); the workgroup scans up to the largest
    int nvl[RG];
    int ncols = 0;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const int r = r0 + 4 * rg + lg;
        nvl[rg] = r < a.n_rows ? max(0, min(a.n_vis[r], a.max_vis)) : 0;
        ncols = max(ncols, nvl[rg]);
    }
    ncols = max(ncols, __shfl_xor(ncols, 16, 64));
    ncols = max(ncols, __shfl_xor(ncols, 32, 64));
    ncols = __builtin_amdgcn_readfirstlane(ncols);
    if (64 * IS_WAVES * (int)blockIdx.x >= ncols) return;   // uniform over the workgroup
    const int Gx = gridDim.x;
    const int wbase = 64 * (IS_WAVES * (int)blockIdx.x + wave);
    constexpr int TSTRIDE = 16;
    const int BSTRIDE = 64 * IS_WAVES * Gx;

    KeyBatch A, B;
    load_batch<false>(kv, req, nullptr, nullptr, 0, ncols, ncols, wbase, TSTRIDE, n, lg, A);   // in flight during the query prep
    {
        // wave w quantises rows w, w + 4, ...; rows past the end copy the last row
        constexpr int PER = R / IS_WAVES;
        QRaw qraw[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) load_query<QBF16>(qraw[j], a.q_idx, min(r0 + wave + IS_WAVES * j, a.n_rows - 1), a.n_heads);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            QRow& qr = sh.q[wave + IS_WAVES * j];
            int sp, mn, mx;
            prep_query<QBF16>(qr, qraw[j], a.w, min(r0 + wave + IS_WAVES * j, a.n_rows - 1), a.n_heads, 0, sp, mn, mx);
            if (l == 0) { qr.spread = sp; qr.smin = mn; qr.smax = mx; }
        }
    }
    if (threadIdx.x == 0) sh.n_fix = 0;
    __syncthreads();

    i32x8 Aq[RG][NM];
    int sa[RG][NM];
    float wl[RG][4 * NM];
    int qsp[RG], qmn[RG], qmx[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
        for (int k = 0; k < NM; ++k) {
            const QRow& q = sh.q[4 * rg + (n >> 2)];
            const int h = 4 * k + (n & 3);
            const uint4 v = *(const uint4*)&q.codes[h][16 * lg];
            Aq[rg][k] = (i32x8){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            sa[rg][k] = q.scales[h][lg];
        }
        const QRow& own = sh.q[4 * rg + lg];
#pragma unroll
        for (int h = 0; h < 4 * NM; ++h) wl[rg][h] = own.w[h];   // 0 above n_heads
        qsp[rg] = own.spread;
        qmn[rg] = own.smin;
        qmx[rg] = own.smax;
    }

    auto compute = [&](const KeyBatch& kb, int col_base) {
#pragma unroll
        for (int t = 0; t < IS_TILES; ++t) {
            const int col0 = col_base + TSTRIDE * t;
            if (col0 >= ncols) break;
            const i32x8 Bk = {(int)kb.code[t].x, (int)kb.code[t].y, (int)kb.code[t].z, (int)kb.code[t].w, 0, 0, 0, 0};
            const uint32_t sd = kb.scl[t];
            const int sb = (int)((sd >> (8 * lg)) & 0xFFu);
            f32x4 d[RG][NM];
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                for (int k = 0; k < NM; ++k) {
                    const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
                    d[rg][k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(Aq[rg][k], Bk, z, 4, 4, 0, sa[rg][k], 0, sb);
                }
            // pin every MFMA in wave-uniform control flow (see the single-row
            // kernel); the results stay in VGPRs (no AGPR reads per tile)
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                for (int k = 0; k < NM; ++k) asm volatile("" : "+v"(d[rg][k]));
            const int b0 = sd & 0xFF, b1 = (sd >> 8) & 0xFF, b2 = (sd >> 16) & 0xFF, b3 = sd >> 24;
            const int kmin = min(min(b0, b1), min(b2, b3)), kmax = max(max(b0, b1), max(b2, b3));
            const int col = col0 + n;
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                const bool ok = (kmax - kmin + qsp[rg] <= 9) && (qmn[rg] + kmin >= 136) && (qmx[rg] + kmax <= 356);
                float acc = 0.0f;
#pragma unroll
                for (int k = 0; k < NM; ++k)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc = fmaf(wl[rg][4 * k + i], relu_bits(d[rg][k][i]), acc);
                acc = (acc == 0.0f) ? 0.0f : acc;
                const bool vis = col < nvl[rg];
                const float val = vis ? acc : -INFINITY;
                const int rl = 4 * rg + lg;                   // the lane's row within the workgroup
                // an 8-block with an unguarded visible key is queued once (lanes 8j + 7)
                if (__builtin_expect(__any(vis && !ok), 0)) {
                    int bad = (vis && !ok) ? 1 : 0;
                    bad |= __builtin_amdgcn_update_dpp(0, bad, 0x111, 0xF, 0xF, false);   // row_shr:1
                    bad |= __builtin_amdgcn_update_dpp(0, bad, 0x112, 0xF, 0xF, false);   // row_shr:2
                    bad |= __builtin_amdgcn_update_dpp(0, bad, 0x114, 0xF, 0xF, false);   // row_shr:4
                    if ((n & 7) == 7 && bad) {
                        const int slot = atomicAdd(&sh.n_fix, 1);
                        sh.fix_col[slot] = col & ~7;
                        sh.fix_row[slot] = (uint8_t)rl;
                    }
                }
                const int64_t r = r0 + rl;
                const bool row_ok = r < a.n_rows;
                if (a.scores && row_ok && col < ((nvl[rg] + 7) & ~7)) a.scores[r * a.scores_stride + col] = val;
                if (a.block_max) {
                    float bm = dpp_row_shr_max(val, 1);
                    bm = dpp_row_shr_max(bm, 2);
                    bm = dpp_row_shr_max(bm, 4);
                    if (row_ok && (n & 7) == 7 && (col & ~7) < nvl[rg]) a.block_max[r * a.block_max_stride + (col >> 3)] = bm;
                }
            }
        }
    };

    // the next batch is always requested (past the end its columns are clamped
    // into range and not used), so every wait names one batch exactly
    for (int b = 0; b < SR_ITERS; b += 2) {
        const int c_a = wbase + b * BSTRIDE, c_b = c_a + BSTRIDE;
        load_batch<false>(kv, req, nullptr, nullptr, 0, ncols, ncols, c_b, TSTRIDE, n, lg, B);
        compute(A, c_a);
        load_batch<false>(kv, req, nullptr, nullptr, 0, ncols, ncols, c_b + BSTRIDE, TSTRIDE, n, lg, A);
        compute(B, c_b);
    }

    // ---- exact path for the queued (row, 8-block)s
    __syncthreads();
    const int nfix = sh.n_fix;
    for (int i = threadIdx.x; i < nfix; i += blockDim.x) {
        const int c8 = sh.fix_col[i], rl = sh.fix_row[i];
        const int64_t r = r0 + rl;
        const int nv = max(0, min(a.n_vis[r], a.max_vis));
        const QRow& q = sh.q[rl];
        float bm = -INFINITY;
        for (int j = 0; j < 8 && c8 + j < nv; ++j) {
            const int64_t e = entry_of(kv, req, c8 + j);
            const float v = exact_key_score(q.codes, q.scales, q.w, a.n_heads, kv.idx_codes + e * 64, kv.idx_scales + e * 4);
            if (a.scores) a.scores[r * a.scores_stride + c8 + j] = v;
            bm = fmaxf(bm, v);
        }
        if (a.block_max) a.block_max[r * a.block_max_stride + (c8 >> 3)] = bm;
    }
}

template <bool QBF16, bool POOL, bool MULTI = false, bool PTE = false>
static void launch_nm(int nm, dim3 grid, dim3 block, hipStream_t st, const KvView& kv, const IndexScoreArgs& a) {
    switch (nm) {
        case 1: hipLaunchKernelGGL((index_score_kernel<QBF16, POOL, 1, MULTI, PTE>), grid, block, 0, st, kv, a); break;
        case 2: hipLaunchKernelGGL((index_score_kernel<QBF16, POOL, 2, MULTI, PTE>), grid, block, 0, st, kv, a); break;
        case 3: hipLaunchKernelGGL((index_score_kernel<QBF16, POOL, 3, MULTI, PTE>), grid, block, 0, st, kv, a); break;
        case 4: hipLaunchKernelGGL((index_score_kernel<QBF16, POOL, 4, MULTI, PTE>), grid, block, 0, st, kv, a); break;
        default: hipLaunchKernelGGL((index_score_heads_kernel<QBF16, POOL, MULTI, PTE>), grid, block, 0, st, kv, a); break;
    }
}

template <bool QBF16>
static void launch_full(bool multi, bool paged, int nm, dim3 grid, dim3 block, hipStream_t st, const KvView& kv,
                        const IndexScoreArgs& a) {
    if (multi) {
        if (paged) launch_nm<QBF16, false, true, true>(nm, grid, block, st, kv, a);
        else launch_nm<QBF16, false, true, false>(nm, grid, block, st, kv, a);
    } else {
        if (paged) launch_nm<QBF16, false, false, true>(nm, grid, block, st, kv, a);
        else launch_nm<QBF16, false, false, false>(nm, grid, block, st, kv, a);
    }
}

template <bool QBF16>
static void launch_shared_nm(int nm, dim3 grid, dim3 block, hipStream_t st, const KvView& kv, const IndexScoreArgs& a,
                             int req) {
    switch (nm) {
        case 1: hipLaunchKernelGGL((index_score_shared_kernel<QBF16, 1, 4>), grid, block, 0, st, kv, a, req); break;
        case 2: hipLaunchKernelGGL((index_score_shared_kernel<QBF16, 2, 4>), grid, block, 0, st, kv, a, req); break;
        case 3: hipLaunchKernelGGL((index_score_shared_kernel<QBF16, 3, 2>), grid, block, 0, st, kv, a, req); break;
        default: hipLaunchKernelGGL((index_score_shared_kernel<QBF16, 4, 2>), grid, block, 0, st, kv, a, req); break;
    }
}

hipError_t launch_index_score_shared(const KvView& kv, const IndexScoreArgs& a, int req, hipStream_t st) {
    const int nm = (a.n_heads + 3) / 4;
    const int rows_per_wg = nm <= 2 ? 16 : 8;
    const dim3 grid((unsigned)((a.max_vis + SR_CHUNK - 1) / SR_CHUNK), (unsigned)((a.n_rows + rows_per_wg - 1) / rows_per_wg)),
        block(IS_WAVES * 64);
    if (a.q_bf16) launch_shared_nm<true>(nm, grid, block, st, kv, a, req);
    else launch_shared_nm<false>(nm, grid, block, st, kv, a, req);
    return hipGetLastError();
}

hipError_t launch_index_score(const KvView& kv, const IndexScoreArgs& a, hipStream_t st) {
    const bool pool = a.pool != nullptr;
    const int cols = pool ? 8 * 2048 : a.max_vis;
    const int nm = (a.n_heads + 3) / 4;
    // A full scan gives a row at most IS_MAX_SLICES slices per workgroup and
    // otherwise as many workgroups as one slice each needs, or fewer while
    // the grid still has about 2,048 of them: rows far shorter than max_vis
    // then leave few workgroups with nothing to do.
    const int chunks = (cols + IS_CHUNK - 1) / IS_CHUNK;
    int gx = chunks;
    if (!pool) {
        const int per_row = (2048 + a.n_rows - 1) / a.n_rows;
        gx = std::min(chunks, std::max((chunks + IS_MAX_SLICES - 1) / IS_MAX_SLICES, per_row));
    }
    if ((chunks + gx - 1) / gx > IS_MAX_SLICES) return hipErrorInvalidValue;   // the fix queue holds 8 slices
    const dim3 grid((unsigned)gx, (unsigned)a.n_rows), block(IS_WAVES * 64);
    if (a.q_bf16) {
        if (pool) launch_nm<true, true>(nm, grid, block, st, kv, a);
        else launch_full<true>(gx < chunks, kv.page_shift >= 0, nm, grid, block, st, kv, a);
    } else {
        if (pool) launch_nm<false, true>(nm, grid, block, st, kv, a);
        else launch_full<false>(gx < chunks, kv.page_shift >= 0, nm, grid, block, st, kv, a);
    }
    return hipGetLastError();
}

}  // namespace csa2
