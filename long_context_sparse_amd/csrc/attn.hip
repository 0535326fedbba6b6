// attn.hip -- K4/K5: sparse attention over the selected FP4 entries, jointly
// with the 8-bit sliding window and an optional sink (gfx950).
//
// Shared-KV MQA: every selected compressed entry is both key and value, and
// the query heads attend in the 512-channel latent space (absorbed query)
// ['DeepSeek-V4' paper page, section 2.3.1 "Shared Key-Value MQA"; MLA article,
// key-weight and deferred value absorption].  The FP4 main entries are
// restored before the matmuls.  The sliding-window entries join the same
// softmax, and an optional per-head sink adds exp(z'_h) to the denominator
// [section 2.3.3].
//
// MI355X mapping
//   * A row's entry list is its selected FP4 entries padded to a multiple of
//     64, then its window entries; it is walked in chunks of 64 with an
//     online softmax.  Every 3 chunks form a unit (at most 4 per row; 12
//     chunks for the dense rows of the heavily compressed branch, so a long
//     row leaves one partial per 768 entries) whose max, sum and output start
//     afresh; the units are joined left to right by one fold.  One workgroup takes (row, group of 16 heads, split):
//     without a workspace there is one split, which folds its units as it
//     goes and writes the final output; with one, a launch with few rows
//     gives each (row, group) up to 4 splits of consecutive units (so the
//     grid reaches about 256 workgroups), each writes its units' partials,
//     and attn_merge_kernel folds them in unit order (then joins, in the
//     two-call form, the other branch's partial, and the sink) with the same
//     operations.  A row's result therefore depends neither on the other
//     rows of the call nor on the split count: the bitwise batch invariance
//     of the decode step ['DeepSeek-V4' page, section 3.3, "Batch
//     Invariance": a split form keeps the accumulation order of the
//     single-workgroup form].  Workgroups are numbered so that a row's
//     workgroups share one XCD and its gathered entries one L2.
//   * 8 waves: wave w dequantises entries 16(w%4)..+15 of the chunk over the
//     channel half w/4 straight into registers as the A operand of
//     S^T = K q^T (V_MFMA_F32_16X16X32_F16), and stores the same values
//     row-major into LDS.  The two half-sums of each S^T tile meet in LDS;
//     every wave then holds all 64 scores of its 16 heads, runs the same
//     softmax in base 2, and keeps P in registers as the B operand of
//     O^T = V^T P^T over its own 64 channels, with V^T read from the
//     row-major LDS copy by transposing reads (DS_READ_B64_TR_B16).
//   * LDS and the partial scores are double-buffered and the next chunk's
//     bytes are in flight while the current one is processed: one barrier
//     per chunk.
//   * Both matmuls run in fp16 with exact operands: the query is scaled by a
//     power of two per head so its largest component sits in [2^14, 2^15).
//     Selected entries carry the fixed factor 2^4: FP4 x E4M3 values have at
//     most 6 significant bits and lie in [2^-10, 2688], so times 2^4 they are
//     normal fp16 numbers, exact, below 65504.  Window entries carry their
//     row's own factor 2^tw, chosen so that the row's largest window group
//     reaches the top of the fp16 range: E4M3 x 2^e values are exact for
//     every group within 22 octaves of it.  The scaled conversion
//     instructions (V_CVT_SCALEF32_PK_F16_FP4 / _FP8) apply the power of two
//     as they convert.  The scalings are undone on the fp32 scores and
//     outputs; a running output that crosses from selected to window chunks
//     is rescaled by 2^(tw - 4) at the crossing (exact in fp32).
#include <atomic>
#include <type_traits>

#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int AT_ENT = 64;              // entries per chunk
constexpr int AT_WAVES = 8;
constexpr int AT_THREADS = 64 * AT_WAVES;
// fp16 elements per entry row of V in LDS: a 16-B pad halves the bank
// conflicts of the 32-B pad (measured: 0.39 against 0.76 conflict cycles per
// active LDS cycle; a 64-B pad 2.4)
constexpr int V_LD = 512 + 8;
constexpr int AT_MAX_SEL = 512;
constexpr int AT_UNIT = 3;              // chunks per unit of the fixed fold
constexpr int AT_UNIT_DENSE = 12;       // chunks per unit of a dense row (one partial per 768 entries)
constexpr int AT_MAX_UNITS = (AT_MAX_SEL / AT_ENT + 128 / AT_ENT + AT_UNIT - 1) / AT_UNIT;   // 4
constexpr int AT_MAX_SPLITS = AT_MAX_UNITS;   // workgroups sharing one (row, head group)
constexpr int AT_TW_SEL = 4;            // power of two on every dequantised selected entry
// bounds of the window's power of two: the crossing factor 2^(tw - AT_TW_SEL)
// and its inverse stay normal fp32 numbers
constexpr int AT_TW_WIN_MIN = -120, AT_TW_WIN_MAX = 100;

struct AttnSmem {
    _Float16 v[2][AT_ENT * V_LD];       // the chunk's dequantised entries [entry][channel], double-buffered
    f32x4 sp[2][AT_WAVES][64];          // per-wave half-channel S^T tiles, double-buffered
    int64_t ent[AT_MAX_SEL];            // cache slot of each selected entry
    float qmax[2][16];                  // per channel half and head: largest |q|
    int wrange[AT_WAVES];               // per wave: largest nonzero window scale code
};
constexpr size_t AT_LDS = sizeof(AttnSmem);
static_assert(AT_LDS <= 160 * 1024, "attention LDS exceeds the 160 KB of a CU");


// Raw bytes of one lane's share of a chunk: the 64 channels
// 256*kh + 64*g .. +63 of one entry (32 B of FP4 codes or 64 B of E4M3 codes)
// and the 4 scale bytes of those channels.
struct RawChunk {
    uint4 c[4];
    uint32_t s;
};

template <bool DENSE>
__device__ __forceinline__ void load_raw(const KvView& kv, const AttnArgs& a, const AttnSmem& sm, int c, int csp,
                                         int nsp, int nsw, int64_t swa0, int req, int et, int kh, int n, int g,
                                         RawChunk& r) {
    // Addresses are selected, the loads are issued unconditionally (the
    // selected-entry case re-reads its 32 code bytes for c[2..3], unused).
    // DENSE: the row's entry e is its position e (every visible entry).
    const bool sel = c < csp;
    int e = 16 * et + n + 64 * (sel ? c : c - csp);
    e = e < (sel ? nsp : nsw) ? e : 0;                // padding lanes re-read entry 0 (masked later)
    const uint8_t* cp;
    const uint8_t* sp;
    if (sel) {
        const int64_t slot = DENSE ? entry_of(kv, req, e) : sm.ent[e];
        cp = kv.main_codes + slot * 256 + 128 * kh + 32 * g;
        sp = kv.main_scales + slot * 32 + 16 * kh + 4 * g;
    } else {
        const int64_t slot = swa0 + e;
        cp = a.swa_codes + slot * 512 + 256 * kh + 64 * g;
        sp = a.swa_scales + slot * 32 + 16 * kh + 4 * g;
    }
    const uint4* p = (const uint4*)cp;
    const uint4* p2 = (const uint4*)(cp + (sel ? 0 : 32));
    r.c[0] = p[0];
    r.c[1] = p[1];
    r.c[2] = p2[0];
    r.c[3] = p2[1];
    r.s = *(const uint32_t*)sp;
}

// Selected entry: dequantise the lane's 64 channels into the QK A operand
// and into V^T, both fp16 and both carrying the exact factor 2^AT_TW_SEL.
// V_CVT_SCALEF32_PK_F16_FP4 expands two E2M1 codes (low nibble first) times
// the power of two of its f32 scale operand, here 2^(AT_TW_SEL + 8); the
// E4M3 scale byte shifted into fp16 position reads as scale * 2^-8 (normal
// and subnormal alike) and one packed fp16 multiply applies it.  FP4 x E4M3
// values have at most 6 significant bits and lie in [2^-10, 2688], so times
// 2^4 they are normal fp16 numbers (at most 43008): exact for every input.
// K-step ks holds channels 8ks .. 8ks+7 of the lane and is also stored to the
// entry's row in LDS at vrow + 8ks.
__device__ __forceinline__ void dequant_main(const RawChunk& r, float cvt_scale, _Float16* vrow, f16x8* kop) {
    const uint32_t words[8] = {r.c[0].x, r.c[0].y, r.c[0].z, r.c[0].w, r.c[1].x, r.c[1].y, r.c[1].z, r.c[1].w};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const uint32_t s16 = ((r.s >> (8 * (ks >> 1))) & 0x7Fu) << 7;
        const f16x2 s2 = __builtin_bit_cast(f16x2, s16 | (s16 << 16));
        f16x2 hp[4];
        hp[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(words[ks], cvt_scale, 0) * s2;
        hp[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(words[ks], cvt_scale, 1) * s2;
        hp[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(words[ks], cvt_scale, 2) * s2;
        hp[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(words[ks], cvt_scale, 3) * s2;
        kop[ks] = (f16x8){hp[0][0], hp[0][1], hp[1][0], hp[1][1], hp[2][0], hp[2][1], hp[3][0], hp[3][1]};
        *(f16x8*)(vrow + 8 * ks) = kop[ks];
    }
}

// Window entry: E4M3 codes times the E8M0 scale 2^e of their 16 channels,
// times the row's window factor 2^tw, in fp16 (V_CVT_SCALEF32_PK_F16_FP8
// converts two E4M3 bytes and multiplies by the power of two of its f32
// scale operand).  E4M3 * 2^(e + tw) is exact in fp16 while
// -15 <= e + tw <= 7; the row's largest group sits at e + tw = 7 (unless the
// window is tinier than 2^-85), groups more than 133 octaves below it
// convert to zero.
__device__ __forceinline__ void dequant_swa(const RawChunk& r, int tw, _Float16* vrow, f16x8* kop) {
    const uint32_t words[16] = {r.c[0].x, r.c[0].y, r.c[0].z, r.c[0].w, r.c[1].x, r.c[1].y, r.c[1].z, r.c[1].w,
                                r.c[2].x, r.c[2].y, r.c[2].z, r.c[2].w, r.c[3].x, r.c[3].y, r.c[3].z, r.c[3].w};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        int ef = (int)((r.s >> (8 * (ks >> 1))) & 0xFFu) + tw;    // biased exponent of 2^(e + tw)
        ef = ef < 0 ? 0 : (ef > 254 ? 254 : ef);                   // e + tw <= 7: the upper clamp is never reached
        const float sc = __uint_as_float((uint32_t)ef << 23);
        f16x2 b[4];
        b[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(words[2 * ks], sc, false);
        b[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(words[2 * ks], sc, true);
        b[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(words[2 * ks + 1], sc, false);
        b[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(words[2 * ks + 1], sc, true);
        kop[ks] = (f16x8){b[0][0], b[0][1], b[1][0], b[1][1], b[2][0], b[2][1], b[3][0], b[3][1]};
        *(f16x8*)(vrow + 8 * ks) = kop[ks];
    }
}

// q B operand of a lane: head h, channels 256*kh + 64*g + 8ks .. +7, ks = 0..7,
// as bf16 (an fp32 query is rounded to nearest even), and the lane's largest
// magnitude.
template <bool QBF16>
__device__ __forceinline__ float load_q_operand(const void* q, int64_t qrow, int kh, int g, bf16x8* qv) {
    const int64_t off = qrow * 512 + 256 * kh + 64 * g;
    float amax = 0.0f;
    if (QBF16) {
        const bf16x8* p = (const bf16x8*)((const uint16_t*)q + off);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qv[ks] = p[ks];
    } else {
        const float4* p = (const float4*)((const float*)q + off);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const float4 x0 = p[2 * ks], x1 = p[2 * ks + 1];
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            uint32_t b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) b[i] = f32_to_bf16_rne(xs[2 * i]) | (f32_to_bf16_rne(xs[2 * i + 1]) << 16);
            qv[ks] = __builtin_bit_cast(bf16x8, make_uint4(b[0], b[1], b[2], b[3]));
        }
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const uint4 u = __builtin_bit_cast(uint4, qv[ks]);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            amax = fmaxf(amax, fabsf(__uint_as_float(w[i] << 16)));
            amax = fmaxf(amax, fabsf(__uint_as_float(w[i] & 0xFFFF0000u)));
        }
    }
    return amax;
}

// The fp16 copy of the query for the selected entries: q * 2^kq with
// 2^14 <= amax * 2^kq < 2^15, so the head's largest component keeps full
// precision and the whole head stays in fp16 range (components below
// amax * 2^-29 lose bits, far below the attention tolerance).
__device__ __forceinline__ void q_to_f16(const bf16x8* qv, int kq, f16x8* qh) {
    const float f = __uint_as_float((uint32_t)(127 + kq) << 23);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const uint4 u = __builtin_bit_cast(uint4, qv[ks]);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
        f16x8 h;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            h[2 * i] = (_Float16)(__uint_as_float(w[i] << 16) * f);
            h[2 * i + 1] = (_Float16)(__uint_as_float(w[i] & 0xFFFF0000u) * f);
        }
        qh[ks] = h;
    }
}

// V^T A operand of P.V for channels ch0 .. ch0+15, contraction step u, read
// from V [entry][channel] with DS_READ_B64_TR_B16.  Within each 16-lane group
// the transposing read hands lane 4a+b element b of the 4-element rows
// addressed by lanes a, a+4, a+8, a+12; lane i of group g addresses entry
// base + i/4, channels ch0 + 4(i%4) .. +3, so lane j receives channel ch0 + j
// of entries base .. base+3.  Two reads fill the 8 slots of group g: entries
// {32u + 4g .. +3} and {32u + 16 + 4g .. +3} (the slots of P^T).
__device__ __forceinline__ f16x8 v_operand(const _Float16* vb, int ch0, int u, int n, int g) {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const int off = (32 * u + 4 * g + (n >> 2)) * V_LD + ch0 + 4 * (n & 3);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + off));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + off + 16 * V_LD));
    const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(f16x8, make_uint4(a.x, a.y, b.x, b.y));
}

// Block -> (row, head group): the workgroups are dealt to the XCDs in turn,
// so block b runs on XCD b % 8; number the (row, group) pairs so that each
// XCD receives a consecutive run of them (a row's groups share an L2).
__device__ __forceinline__ int xcd_order(int b, int total) {
    const int x = b & 7, k = b >> 3;
    int base = 0;
    for (int y = 0; y < x; ++y) base += (total - y + 7) >> 3;
    return base + k;
}

// Units of a row's entry list: ceil(chunks / 3) (dense rows: ceil(chunks /
// 12)), chunks = ceil(selected / 64) + ceil(window / 64).
__device__ __forceinline__ int row_units(const AttnArgs& a, int nsp_raw, int nsw_raw) {
    const int nsp = a.dense_n ? min(max(nsp_raw, 0), a.max_dense) : (a.idx ? min(max(nsp_raw, 0), AT_MAX_SEL) : 0);
    const int nsw = a.swa_codes ? min(max(nsw_raw, 0), 128) : 0;
    const int ctot = (nsp + AT_ENT - 1) / AT_ENT + (nsw + AT_ENT - 1) / AT_ENT;
    const int unit = a.dense_n ? AT_UNIT_DENSE : AT_UNIT;
    return (ctot + unit - 1) / unit;
}

// The fold of one unit (base-2 max m, sum l, output o = sum of 2^(z - m) E,
// unnormalised) into the running (M, L, O), in unit order:
//   M' = max(M, m),  L' = 2^(m - M') l + 2^(M - M') L,  O' likewise.
// attn_kernel and attn_merge_kernel both call these two functions, with
// explicit fma so that no contraction differs between them.
struct FoldW { float wa, wb; };
__device__ __forceinline__ FoldW fold_unit(float& M, float& L, float m, float l) {
    const float Mn = fmaxf(M, m);
    const float wa = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
    const float wb = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - Mn);
    L = fmaf(wb, l, wa * L);
    M = Mn;
    return {wa, wb};
}
__device__ __forceinline__ f32x4 fold_out(const FoldW& f, f32x4 O, f32x4 o) {
    return (f32x4){fmaf(f.wb, o[0], f.wa * O[0]), fmaf(f.wb, o[1], f.wa * O[1]), fmaf(f.wb, o[2], f.wa * O[2]),
                   fmaf(f.wb, o[3], f.wa * O[3])};
}

// The end of a row and head: the folded units (M, L, O), an external partial
// (lse_p, o_in: base-2 log-sum-exp and normalised output) and the sink sk
// (base 2) in one denominator:
//   out = (2^(M - X) O + 2^(lse_p - X) o_in) / (2^(M - X) L + 2^(lse_p - X) + 2^(sk - X)),
// X the largest of the three; lse2 the base-2 log-sum-exp (-inf if empty).
struct FinalW { float wo, wp, inv, lse2; };
__device__ __forceinline__ FinalW final_weights(float M, float L, float lse_p, float sk) {
    const float X = fmaxf(fmaxf(M, lse_p), sk);
    const float wo = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - X);
    const float wp = lse_p == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(lse_p - X);
    const float ws = sk == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sk - X);
    const float den = fmaf(wo, L, wp) + ws;
    const bool empty = X == -INFINITY || den == 0.0f;
    return {wo, wp, empty ? 0.0f : 1.0f / den, empty ? -INFINITY : X + log2f(den)};
}
__device__ __forceinline__ f32x4 final_out(const FinalW& f, f32x4 O, float4 pin) {
    return (f32x4){fmaf(f.wo, O[0], f.wp * pin.x) * f.inv, fmaf(f.wo, O[1], f.wp * pin.y) * f.inv,
                   fmaf(f.wo, O[2], f.wp * pin.z) * f.inv, fmaf(f.wo, O[3], f.wp * pin.w) * f.inv};
}

// SPLIT: the launch has several splits per (row, group) (their partials go to
// the workspace); without it the workgroup folds its units itself, and only
// that form holds the folded output in registers.
template <bool QBF16, bool SPLIT, bool DENSE>
__global__ __launch_bounds__(AT_THREADS) void attn_kernel(KvView kv, AttnArgs a) {
    extern __shared__ __align__(16) uint8_t at_smem[];
    AttnSmem& sm = *(AttnSmem*)at_smem;
    const int G = a.n_heads >> 4, S = a.n_splits;
    const int id = xcd_order(blockIdx.x, a.n_rows * G * S);   // a (row, group)'s splits are consecutive
    const int row = id / (G * S);
    const int hg = (id - row * G * S) / S, split = id - (row * G + hg) * S;
    const int h0 = 16 * hg;
    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int n = l & 15, g = l >> 4;
    const int et = wave & 3, kh = wave >> 2;
    const int nsp = DENSE ? min(max(a.dense_n[row], 0), a.max_dense)
                          : (a.idx ? min(max(a.idx_count[row], 0), AT_MAX_SEL) : 0);
    const int nsw = a.swa_codes ? min(max(a.swa_count[row], 0), 128) : 0;
    constexpr int UNIT = DENSE ? AT_UNIT_DENSE : AT_UNIT;           // chunks per unit
    const int csp = (nsp + AT_ENT - 1) / AT_ENT;
    const int ctot = csp + (nsw + AT_ENT - 1) / AT_ENT;
    const int U = (ctot + UNIT - 1) / UNIT;
    const int ub = split * U / S, ue = (split + 1) * U / S;         // this split's units
    const int cb = UNIT * ub, ce = min(UNIT * ue, ctot);            // and chunks
    if (SPLIT && ue == ub) return;                                  // a short row: no unit here
    const int64_t swa0 = nsw ? a.swa_first[row] : 0;

    // The cache slots of the selected entries (the index is read before its
    // count is known: one dependent load less), the query and its per-head
    // scale, the exponent range of the row's window scales.  Every load is
    // issued before any is used, from a valid address (a dummy one where it is
    // not needed): a load under a branch makes the compiler wait for it where
    // the branch joins, which would put three memory round trips in a row.
    const int32_t* idx_p = (!DENSE && a.idx) ? a.idx + (int64_t)row * a.idx_stride +
                                                   min((int64_t)threadIdx.x, a.idx_stride - 1)
                                             : (const int32_t*)a.q;
    const int32_t idx_raw = *idx_p;
    const int req_r = *(a.req ? a.req + row : (const int32_t*)a.q);
    // the external partial's log-sum-exp and the sink, used by the epilogue
    const float lse_raw = *(a.lse_in ? a.lse_in + (int64_t)row * a.n_heads + h0 + n : (const float*)a.q);
    const float sink_raw = *(a.sink ? a.sink + h0 + n : (const float*)a.q);
    const bool has_sc = (int)threadIdx.x * 8 < nsw * 32;
    const uint2 scv = *(const uint2*)(has_sc ? a.swa_scales + swa0 * 32 + 8 * threadIdx.x : (const uint8_t*)a.q);
    bf16x8 qb[8];
    float qa = load_q_operand<QBF16>(a.q, (int64_t)row * a.n_heads + h0 + n, kh, g, qb);
    if (!DENSE && (int)threadIdx.x < nsp) sm.ent[threadIdx.x] = entry_of(kv, req_r, idx_raw);   // paged: one more load
    qa = max_xor32(max_xor16(qa));
    if (et == 0 && g == 0) sm.qmax[kh][n] = qa;
    // The window's scale range needs the window's position first (two memory
    // round trips, the selected slots one), and only chunks of the window use
    // it: a split whose first chunk is a selected one publishes it at the
    // barrier after that chunk's dequantisation, when the scales have long
    // arrived; one that starts in the window publishes it here.
    const bool early = cb >= csp;
    auto publish_wmax = [&]() __attribute__((always_inline)) {
        int wmax = 0;                               // over nonzero scale codes (all-zero groups have code 0)
        if (has_sc) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int c = (int)(((i < 4 ? scv.x : scv.y) >> (8 * (i & 3))) & 0xFFu);
                if (c) wmax = max(wmax, c);
            }
        }
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) wmax = max(wmax, __shfl_xor(wmax, d, 64));
        if (l == 0) sm.wrange[wave] = wmax;
    };
    if (early) publish_wmax();
    __syncthreads();
    const float qmax = fmaxf(sm.qmax[0][n], sm.qmax[1][n]);
    int kq = qmax > 0.0f ? 14 - ((int)((__float_as_uint(qmax) >> 23) & 0xFFu) - 127) : 0;
    kq = kq < -110 ? -110 : (kq > 110 ? 110 : kq);
    f16x8 qh[8];
    q_to_f16(qb, kq, qh);
    // logits in base 2: z2 = S' * cz with S' = S * 2^(kq + factor), per entry kind
    constexpr float LOG2E = 1.44269504088896341f, LN2 = 0.693147180559945309f;
    const float cz_sel = ldexpf(a.scale * LOG2E, -kq - AT_TW_SEL);
    constexpr float cvt_sel = (float)(1 << (AT_TW_SEL + 8));                    // 2^(AT_TW_SEL + 8)
    // The window's power of two 2^tw: its largest group (biased scale code
    // wmax, e = wmax - 127) lands at e + tw = 7, the top of the exact fp16
    // range; groups within 22 octaves of it are exact, smaller ones rounded
    // (an absolute change of at most 2^-40 of the window's largest value).
    // Selected entries always carry 2^AT_TW_SEL.  cz_win: the window's logit
    // factor; cross: a running output crossing from selected to window chunks
    // is re-expressed by 2^(tw - AT_TW_SEL); pw_win: 2^-tw.
    int tw = 0;
    float cz_win = 0.0f, cross = 1.0f, pw_win = 1.0f;
    auto take_tw = [&]() __attribute__((always_inline)) {
        int wmax = 0;
#pragma unroll
        for (int w = 0; w < AT_WAVES; ++w) wmax = max(wmax, sm.wrange[w]);
        tw = wmax ? 134 - wmax : 0;
        tw = tw < AT_TW_WIN_MIN ? AT_TW_WIN_MIN : (tw > AT_TW_WIN_MAX ? AT_TW_WIN_MAX : tw);
        cz_win = ldexpf(a.scale * LOG2E, -kq - tw);
        cross = __uint_as_float((uint32_t)(127 + tw - AT_TW_SEL) << 23);
        pw_win = __uint_as_float((uint32_t)(127 - tw) << 23);
    };
    if (early) take_tw();

    // Software pipeline, one barrier per chunk: while a wave turns the scores of
    // chunk c into probabilities and accumulates P.V (LDS buffers c & 1), it
    // dequantises chunk c + 1 and computes its partial scores (buffers
    // (c + 1) & 1).  Three chunks are in flight: chunk c's bytes sit in
    // raw[(c - cb) % 3], and right after they are dequantised the loads of
    // chunk c + 3 go into the same registers (a gathered entry takes several
    // microseconds to arrive when every CU is gathering).
    RawChunk raw0, raw1, raw2;
    if (ce > cb) {
        load_raw<DENSE>(kv, a, sm, cb, csp, nsp, nsw, swa0, req_r, et, kh, n, g, raw0);
        load_raw<DENSE>(kv, a, sm, min(cb + 1, ce - 1), csp, nsp, nsw, swa0, req_r, et, kh, n, g, raw1);
        load_raw<DENSE>(kv, a, sm, min(cb + 2, ce - 1), csp, nsp, nsw, swa0, req_r, et, kh, n, g, raw2);
    }
    f32x4 oacc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) oacc[ct] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;            // base-2 running max and sum of the unit
    float neg1 = -1.0f;
    asm volatile("" : "+v"(neg1));                    // opaque to the optimiser (see stage_b)
    const int chb = 256 * kh + 64 * g;               // first of this lane's 64 dequant channels
    const int v_lane = (16 * et + n) * V_LD + chb;  // this lane's entry row and channels in LDS

    // dequantise chunk c, its partial scores into sp[c & 1]; reload raw with chunk c + 3
    auto stage_a = [&](auto swc, const int c, RawChunk& raw) __attribute__((always_inline)) {
        constexpr bool SW = decltype(swc)::value;
        _Float16* vb = sm.v[c & 1];
        f16x8 kop[8];
        if (SW) dequant_swa(raw, tw, vb + v_lane, kop);
        else dequant_main(raw, cvt_sel, vb + v_lane, kop);
        // always issued (near the end they re-read the final chunk, unused): a
        // load under a branch makes the compiler wait for it at the join
        load_raw<DENSE>(kv, a, sm, min(c + 3, ce - 1), csp, nsp, nsw, swa0, req_r, et, kh, n, g, raw);
        f32x4 sc = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[ks], qh[ks], sc, 0, 0, 0);
        sm.sp[c & 1][wave][l] = sc;
    };
    // probabilities of chunk c and O^T += V^T P^T over channels 64*wave .. +63
    auto stage_b = [&](const int c) __attribute__((always_inline)) {
        const int buf = c & 1;
        const int nent = c >= ce ? 0 : min(c < csp ? nsp - 64 * c : nsw - 64 * (c - csp), AT_ENT);
        f32x4 z[4];                                      // z[t][i]: entry 16t + 4g + i, head n
#pragma unroll
        for (int t = 0; t < 4; ++t) z[t] = sm.sp[buf][t][l] + sm.sp[buf][t + 4][l];
        if (nent < AT_ENT) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * t + 4 * g + i >= nent) z[t][i] = -INFINITY;
        }
        // a tree of three-operand maxima (V_MAX3_F32)
        auto mx3 = [](float x, float y, float w) { return fmaxf(fmaxf(x, y), w); };
        const float m9 = mx3(mx3(z[0][0], z[0][1], z[0][2]), mx3(z[0][3], z[1][0], z[1][1]),
                             mx3(z[1][2], z[1][3], z[2][0]));
        const float m7 = mx3(mx3(z[2][1], z[2][2], z[2][3]), mx3(z[3][0], z[3][1], z[3][2]), z[3][3]);
        float m = max_xor32(max_xor16(fmaxf(m9, m7)));
        const bool win = c >= csp;
        const float cz = win ? cz_win : cz_sel;
        const float m_new = fmaxf(m_run, m * cz);         // cz > 0: the scaled maximum
        const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        float lsum = 0.0f;
        // P^T slot 8g + j of step u: entry 32u + 4g + j (j < 4), 32u + 12 + 4g + j.
        // Each probability enters P.V as an fp16 pair, p = hi + lo + O(2^-24 p)
        // (hi = fp16(p); p - hi is exact in fp32): one fp16 P would carry a
        // relative error of 2^-12 into every term of the output, which for
        // entries near the FP4 maximum (2,688) is far above the tolerance.
        f16x8 pb[2], pl[2];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(z[t][i], cz, -m_new));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(z[t][i + 1], cz, -m_new));
                lsum += p0;
                lsum += p1;
                const f16x2 hi = (f16x2){(_Float16)p0, (_Float16)p1};
                // p - hi is exact; as an fma with an opaque -1 (not folded
                // into a subtraction) the compiler forms it from the fp16 hi
                // and the fp32 p with V_FMA_MIX{LO,HI}_F16, one rounding to
                // fp16 written in place: the same bits as an fp32 difference
                // and a conversion, in fewer instructions
                const f16x2 lo = (f16x2){(_Float16)__builtin_fmaf((float)hi[0], neg1, p0),
                                         (_Float16)__builtin_fmaf((float)hi[1], neg1, p1)};
                pb[t >> 1][4 * (t & 1) + i] = hi[0];
                pb[t >> 1][4 * (t & 1) + i + 1] = hi[1];
                pl[t >> 1][4 * (t & 1) + i] = lo[0];
                pl[t >> 1][4 * (t & 1) + i + 1] = lo[1];
            }
        lsum = add_xor32(add_xor16(lsum));
        l_run = l_run * alpha + lsum;
        m_run = m_new;
        const _Float16* vb = sm.v[buf];
        // the first window chunk re-expresses the running output in the
        // window's factor: cross, a power of two, joins alpha in one factor
        // (an exact product unless it falls below the normal range, where the
        // running output no longer counts)
        const float ra = (win && c == csp) ? cross * alpha : alpha;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            f32x4 o = oacc[ct] * ra;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const f16x8 vo = v_operand(vb, 64 * wave + 16 * ct, u, n, g);
                o = __builtin_amdgcn_mfma_f32_16x16x32_f16(vo, pb[u], o, 0, 0, 0);
                o = __builtin_amdgcn_mfma_f32_16x16x32_f16(vo, pl[u], o, 0, 0, 0);
            }
            oacc[ct] = o;
        }
    };
    const std::integral_constant<bool, false> SEL{};
    const std::integral_constant<bool, true> WIN{};
    // One pipeline step: stage A of chunk c + 1 with stage B of chunk c.  The
    // steps run in threes with nothing conditional but the chunk type, so the
    // compiler can count the loads in flight on every path that continues;
    // the last chunk leaves the loop through a branch that issues no load.
    auto step = [&](const int c, RawChunk& next_raw) __attribute__((always_inline)) {
        if (c + 1 < csp) stage_a(SEL, c + 1, next_raw);
        else stage_a(WIN, c + 1, next_raw);
        stage_b(c);
        __syncthreads();
    };

    // The end of unit u, whose last chunk is c_last: with several splits its
    // partial (output without the factor of its last chunk's kind,
    // unnormalised, and its max and sum) goes to the workspace, else it is
    // folded into (Mf, Lf, Of); the next unit starts afresh.
    const int h = h0 + n;
    const float pw_sel = 1.0f / (float)(1 << AT_TW_SEL);                  // 2^-AT_TW_SEL (exact)
    float Mf = -INFINITY, Lf = 0.0f;
    f32x4 Of[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) Of[ct] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    auto end_unit = [&](const int u, const int c_last) __attribute__((always_inline)) {
        const float pw = c_last >= csp ? pw_win : pw_sel;
        if constexpr (SPLIT) {
            const size_t ps = ((size_t)row * a.n_heads + h) * a.max_units + u;
            float* wsO = a.ws;
            float* wsM = wsO + (size_t)a.n_rows * a.n_heads * a.max_units * 512;
            float* wsL = wsM + (size_t)a.n_rows * a.n_heads * a.max_units;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                // partials are written once and read by another kernel:
                // non-temporal stores stream them out instead of leaving them
                // dirty in L2 for the end-of-kernel write-back
                __builtin_nontemporal_store(oacc[ct] * pw, (f32x4*)(wsO + ps * 512 + 64 * wave + 16 * ct + 4 * g));
            if (wave == 0 && g == 0) { wsM[ps] = m_run; wsL[ps] = l_run; }
        } else {
            const FoldW f = fold_unit(Mf, Lf, m_run, l_run);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) Of[ct] = fold_out(f, Of[ct], oacc[ct] * pw);
        }
        m_run = -INFINITY;
        l_run = 0.0f;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) oacc[ct] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    };

    static_assert(AT_UNIT % 3 == 0 && AT_UNIT_DENSE % 3 == 0, "a unit is whole turns of the three-step loop");
    if (ce > cb) {
        if (cb < csp) stage_a(SEL, cb, raw0);
        else stage_a(WIN, cb, raw0);
        if (!early) publish_wmax();
        __syncthreads();
        if (!early) take_tw();
        for (int c = cb;; c += 3) {
            if (c > cb && c % UNIT == 0) end_unit(c / UNIT - 1, c - 1);   // c starts a unit
            if (c + 1 >= ce) { stage_b(c); break; }
            step(c, raw1);
            if (c + 2 >= ce) { stage_b(c + 1); break; }
            step(c + 1, raw2);
            if (c + 3 >= ce) { stage_b(c + 2); break; }
            step(c + 2, raw0);
        }
        end_unit((ce - 1) / UNIT, ce - 1);
    }
    if constexpr (SPLIT) return;
    // ---- epilogue: the folded units, an external partial (o_in, lse_in) and
    // the sink in one denominator; write O^T[64*wave + 16ct + 4g + i][head
    // h0 + n].  Natural-log terms become base 2 with log2(e).
    const float lse_p = a.lse_in ? lse_raw * LOG2E : -INFINITY;
    const float sk = a.sink ? sink_raw * LOG2E : -INFINITY;
    const FinalW fw = final_weights(Mf, Lf, lse_p, sk);
    const float* oin = a.o_in ? a.o_in + ((int64_t)row * a.n_heads + h) * 512 : nullptr;
    float* orow = a.out + ((int64_t)row * a.n_heads + h) * 512;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        const int ch = 64 * wave + 16 * ct + 4 * g;
        const float4 pin = oin ? *(const float4*)(oin + ch) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        __builtin_nontemporal_store(final_out(fw, Of[ct], pin), (f32x4*)(orow + ch));
    }
    if (a.lse_out && wave == 0 && g == 0) a.lse_out[(int64_t)row * a.n_heads + h] = fw.lse2 * LN2;
}

// Folds the unit partials of every (row, head) in unit order, then joins the
// external partial and the sink: the same operations as the epilogue of a
// single-split attn_kernel.  One thread per (row, head, 4 channels).  Sparse
// rows have at most AT_MAX_UNITS units, whose loads are all issued before
// any is used (slots past the row's unit count are read but not folded);
// dense rows walk their units with the next unit's loads in flight.
template <bool DENSE>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
    constexpr float LOG2E = 1.44269504088896341f, LN2 = 0.693147180559945309f;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)a.n_rows * a.n_heads * 128) return;
    const int64_t rh = t >> 7;                        // row * n_heads + head
    const int c4 = (int)(t & 127) * 4;
    const int row = (int)(rh / a.n_heads), h = (int)(rh - (int64_t)row * a.n_heads);
    const int MU = DENSE ? a.max_units : AT_MAX_UNITS;
    const float* wsO = a.ws;
    const float* wsM = wsO + (size_t)a.n_rows * a.n_heads * MU * 512;
    const float* wsL = wsM + (size_t)a.n_rows * a.n_heads * MU;
    const int nsp_raw = DENSE ? a.dense_n[row] : (a.idx ? a.idx_count[row] : 0);
    const int nsw_raw = a.swa_codes ? a.swa_count[row] : 0;
    const float lse_p = a.lse_in ? a.lse_in[rh] * LOG2E : -INFINITY;
    const float sk = a.sink ? a.sink[h] * LOG2E : -INFINITY;
    const float4 pin = a.o_in ? *(const float4*)(a.o_in + rh * 512 + c4) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    const int U = row_units(a, nsp_raw, nsw_raw);
    float M = -INFINITY, L = 0.0f;
    f32x4 O = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (!DENSE) {
        float m[AT_MAX_UNITS], lw[AT_MAX_UNITS];
        f32x4 o[AT_MAX_UNITS];
#pragma unroll
        for (int u = 0; u < AT_MAX_UNITS; ++u) {
            m[u] = wsM[rh * AT_MAX_UNITS + u];
            lw[u] = wsL[rh * AT_MAX_UNITS + u];
            o[u] = *(const f32x4*)(wsO + (rh * AT_MAX_UNITS + u) * 512 + c4);
        }
#pragma unroll
        for (int u = 0; u < AT_MAX_UNITS; ++u) {
            if (u < U) {
                const FoldW f = fold_unit(M, L, m[u], lw[u]);
                O = fold_out(f, O, o[u]);
            }
        }
    } else {
        const int Uc = min(U, MU);
        float mn = 0.0f, ln = 0.0f;
        f32x4 on = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        if (Uc > 0) {
            mn = wsM[rh * MU];
            ln = wsL[rh * MU];
            on = *(const f32x4*)(wsO + (rh * MU) * 512 + c4);
        }
        for (int u = 0; u < Uc; ++u) {
            const float mu = mn, lu = ln;
            const f32x4 ou = on;
            const int un = min(u + 1, Uc - 1);        // the next unit's loads (the last one re-reads itself)
            mn = wsM[rh * MU + un];
            ln = wsL[rh * MU + un];
            on = *(const f32x4*)(wsO + (rh * MU + un) * 512 + c4);
            const FoldW f = fold_unit(M, L, mu, lu);
            O = fold_out(f, O, ou);
        }
    }
    const FinalW fw = final_weights(M, L, lse_p, sk);
    __builtin_nontemporal_store(final_out(fw, O, pin), (f32x4*)(a.out + rh * 512 + c4));
    if (a.lse_out && c4 == 0) a.lse_out[rh] = fw.lse2 * LN2;
}

int attn_splits(int n_rows, int n_heads) {
    const int groups = n_rows * (n_heads >> 4);
    if (groups <= 0) return 1;
    const int s = 256 / groups;                       // fill the 256 CUs, one workgroup each
    return s < 2 ? 1 : (s > AT_MAX_SPLITS ? AT_MAX_SPLITS : s);
}

// one partial per unit, whatever the split count
size_t attn_workspace_bytes(int n_rows, int n_heads, int n_splits) {
    if (n_splits <= 1) return 0;
    return (size_t)n_rows * n_heads * AT_MAX_UNITS * (512 + 2) * sizeof(float);
}

// Dense rows of up to max_dense entries: units of the longest row, and the
// splits that fill the 256 CUs once (at most one per unit).
int dense_units(int max_dense) {
    const int chunks = (max_dense + AT_ENT - 1) / AT_ENT + 128 / AT_ENT;
    return (chunks + AT_UNIT_DENSE - 1) / AT_UNIT_DENSE;
}

int dense_splits(int n_rows, int n_heads, int max_dense) {
    const int groups = n_rows * (n_heads >> 4);
    if (groups <= 0) return 1;
    const int s = 256 / groups, u = dense_units(max_dense);
    return s < 2 ? 1 : (s > u ? u : s);
}

size_t dense_workspace_bytes(int n_rows, int n_heads, int max_dense) {
    if (dense_splits(n_rows, n_heads, max_dense) <= 1) return 0;
    return (size_t)n_rows * n_heads * dense_units(max_dense) * (512 + 2) * sizeof(float);
}

// The kernels' dynamic LDS above 64 KB is allowed once per device (the flag
// per device is set only after every attribute succeeded; a race between two
// host threads on a new device repeats the same idempotent calls).
constexpr int AT_MAX_DEVICES = 64;
static std::atomic<bool> g_attr_set[AT_MAX_DEVICES];

static hipError_t set_lds_attrs() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool cached = dev >= 0 && dev < AT_MAX_DEVICES;
    if (cached && g_attr_set[dev].load(std::memory_order_acquire)) return hipSuccess;
    const void* kernels[8] = {
        (const void*)attn_kernel<true, false, false>, (const void*)attn_kernel<false, false, false>,
        (const void*)attn_kernel<true, true, false>,  (const void*)attn_kernel<false, true, false>,
        (const void*)attn_kernel<true, false, true>,  (const void*)attn_kernel<false, false, true>,
        (const void*)attn_kernel<true, true, true>,   (const void*)attn_kernel<false, true, true>};
    for (const void* k : kernels)
        if ((e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)AT_LDS)) != hipSuccess) return e;
    if (cached) g_attr_set[dev].store(true, std::memory_order_release);
    return hipSuccess;
}

template <bool DENSE>
static hipError_t launch_attn_kind(const KvView& kv, const AttnArgs& a, hipStream_t st) {
    const unsigned blocks = (unsigned)a.n_rows * (unsigned)(a.n_heads >> 4) * (unsigned)a.n_splits;
    const bool split = a.n_splits > 1;
    if (a.q_bf16 && split) hipLaunchKernelGGL((attn_kernel<true, true, DENSE>), dim3(blocks), dim3(AT_THREADS), AT_LDS, st, kv, a);
    else if (a.q_bf16) hipLaunchKernelGGL((attn_kernel<true, false, DENSE>), dim3(blocks), dim3(AT_THREADS), AT_LDS, st, kv, a);
    else if (split) hipLaunchKernelGGL((attn_kernel<false, true, DENSE>), dim3(blocks), dim3(AT_THREADS), AT_LDS, st, kv, a);
    else hipLaunchKernelGGL((attn_kernel<false, false, DENSE>), dim3(blocks), dim3(AT_THREADS), AT_LDS, st, kv, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !split) return e;
    const int64_t threads = (int64_t)a.n_rows * a.n_heads * 128;
    hipLaunchKernelGGL((attn_merge_kernel<DENSE>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_attn(const KvView& kv, const AttnArgs& a_in, size_t ws_bytes, hipStream_t st) {
    hipError_t e = set_lds_attrs();
    if (e != hipSuccess) return e;
    AttnArgs a = a_in;
    a.dense_n = nullptr;
    a.max_units = AT_MAX_UNITS;
    a.n_splits = attn_splits(a.n_rows, a.n_heads);
    if (!a.ws || ws_bytes < attn_workspace_bytes(a.n_rows, a.n_heads, a.n_splits)) a.n_splits = 1;
    return launch_attn_kind<false>(kv, a, st);
}

hipError_t launch_attn_dense(const KvView& kv, const AttnArgs& a_in, size_t ws_bytes, hipStream_t st) {
    hipError_t e = set_lds_attrs();
    if (e != hipSuccess) return e;
    AttnArgs a = a_in;
    a.idx = nullptr;
    a.max_units = dense_units(a.max_dense);
    a.n_splits = dense_splits(a.n_rows, a.n_heads, a.max_dense);
    if (!a.ws || ws_bytes < dense_workspace_bytes(a.n_rows, a.n_heads, a.max_dense)) a.n_splits = 1;
    return launch_attn_kind<true>(kv, a, st);
}

}  // namespace csa2
