// topk.hip -- K3: exact row-wise top-k (gfx950).
//
// Top-k selector of the lightning indexer ['DeepSeek-V4' paper page, section
// 2.3.1] and the block-pool step of the hierarchical sparse indexer (groups
// of 8 positions ranked by their maximum, up to 2,048 kept; V4.1-Flash
// architecture page).  Rank = (key descending, column ascending); columns
// are in id order, so ties go to the lower position / block.
//
// One 1024-thread workgroup per row.  Keys become order-preserving 32-bit
// integers (-inf = 0 = absent).  The bits above the highest bit in which the
// smallest and the largest present key differ are common to every key and
// are skipped; an MSB-first radix select then resolves 12, 10 and 10 bits per
// pass with an LDS histogram of 4,096 bins (scores of one row share few
// exponent values, so a digit that covers only exponent bits would send most
// atomics to one bin; 12 bits reach into the mantissa), and stops as soon as
// the bin holding the k-th key is taken whole, or holds at most 64 keys:
// those are listed and ranked directly.  A block-wide scan in column
// order writes the selected ids ascending.  Thread t owns columns
// [16t, 16t+16) of each 16,384-column sweep, so column order is thread order,
// then item order.  Rows of at most 16,384 columns stay in registers; longer
// rows are re-read.  A row held in registers first bounds its k-th key from
// below by one radix pass over the maxima of groups of 8 columns (the k
// largest group maxima are k distinct keys) and drops the keys under that
// bin before the selection proper.
//
// Wave-level scans and reductions use DPP row shifts and row broadcasts (no
// LDS round trips); the 16 wave totals meet in LDS behind one barrier, and
// every thread forms its own prefix from them.  A radix pass costs three
// barriers.
//
// The Full layer's two selections (2,048 blocks by their maxima, then 512
// positions among those blocks' scores) run fused in one workgroup per row,
// with the pool kept in LDS between them, or, for launches of few long rows,
// side by side in two workgroups per row: the top 512 positions lie in the
// top 512 blocks, so they are selected from the blocks at or above a radix
// bin of the block maxima without waiting for the pool.  A row whose blocks
// all fit the pool takes its top k directly among its scores.
#include "csa2.h"
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

constexpr int TK_THREADS = 1024;
constexpr int TK_ITEMS = 16;
constexpr int TK_SWEEP = TK_THREADS * TK_ITEMS;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_BINS = 4096;
constexpr int TK_POOL = 2048;
static_assert(CSA2_MAX_SELECT <= TK_BINS, "selected ids are staged in the histogram");
static_assert(CSA2_MAX_POOL_BLOCKS <= TK_POOL, "the pool is held in LDS");

struct __align__(16) TkShared {
    uint32_t hist[TK_BINS];
    uint32_t part[2][TK_WAVES];
    uint32_t red[3][TK_WAVES];
    uint32_t digit, above, count, digit2;
    uint32_t ovf[TK_WAVES];            // split selection: a wave had more candidate blocks than its list holds
    uint32_t lcnt;                     // keys of the k-th key's bin, once it holds at most 64 (ranked directly)
    uint32_t lkey[64];
    int32_t lcol[64];
    int32_t pool[TK_POOL];             // fused selection: the row's pool, ascending
};

// ---------------------------------------------------------------- wave primitives
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t x, uint32_t identity) {
    return __builtin_amdgcn_update_dpp(identity, x, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive scan (sum) over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
    x += dpp<0x111>(x, 0u);            // row_shr:1
    x += dpp<0x112>(x, 0u);            // row_shr:2
    x += dpp<0x114>(x, 0u);            // row_shr:4
    x += dpp<0x118>(x, 0u);            // row_shr:8
    x += dpp<0x142, 0xA>(x, 0u);       // row_bcast:15 into rows 1 and 3
    x += dpp<0x143, 0xC>(x, 0u);       // row_bcast:31 into rows 2 and 3
    return x;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
    x = max(x, dpp<0x111>(x, 0u));
    x = max(x, dpp<0x112>(x, 0u));
    x = max(x, dpp<0x114>(x, 0u));
    x = max(x, dpp<0x118>(x, 0u));
    x = max(x, dpp<0x142, 0xA>(x, 0u));
    x = max(x, dpp<0x143, 0xC>(x, 0u));
    return __builtin_amdgcn_readlane(x, 63);
}

__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
    x = min(x, dpp<0x111>(x, 0xFFFFFFFFu));
    x = min(x, dpp<0x112>(x, 0xFFFFFFFFu));
    x = min(x, dpp<0x114>(x, 0xFFFFFFFFu));
    x = min(x, dpp<0x118>(x, 0xFFFFFFFFu));
    x = min(x, dpp<0x142, 0xA>(x, 0xFFFFFFFFu));
    x = min(x, dpp<0x143, 0xC>(x, 0xFFFFFFFFu));
    return __builtin_amdgcn_readlane(x, 63);
}

// Exclusive scan of v over the workgroup in thread order; `total` gets the
// sum.  One barrier; part[buf] must not be in use by a previous scan.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* part, uint32_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t incl = wave_incl_sum(v);
    if (lane == 63) part[wave] = incl;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < TK_WAVES; ++w) {
        const uint32_t p = part[w];
        before += (w < wave) ? p : 0u;
        tot += p;
    }
    total = tot;
    return before + incl - v;
}

// ---------------------------------------------------------------- one row's selection
// KEYS(sweep, u) fills u[16] with the order keys of columns
// sweep*16384 + 16*threadIdx.x + i (0 where absent); EMIT(col, slot, mark)
// records selected column `col` for output slot `slot`; with MARK, `mark` is
// 1 where the column's key passes (u & thr_mask) >= thr_val below (else it
// is 0).  Returns the count.
// NSW = 1 compiles the case of one sweep (ncols <= 16,384: the keys are read
// once and stay in registers); NSW = 0 handles any ncols.
//
// With 0 < k2 < k, the first radix pass also locates the histogram bin of the
// k2-th largest key, and (thr_mask, thr_val) are set so that the keys u with
// (u & thr_mask) >= thr_val are those of that bin and above: a superset of
// the top k2.  Otherwise every key passes (thr_mask = thr_val = 0).
//
// HINT (one sweep only): every present key lies in [hint_min, hint_max] and
// the histogram is already clear, so the opening count / min / max round is
// skipped; the count of present keys comes from the first pass's histogram.
//
// nit (wave-uniform, one sweep only): items nit .. 15 of every thread of the
// wave are absent, so the passes over a thread's items stop there (each
// instruction a thread runs costs the workgroup 16 cycles of VALU issue).
template <int NSW, class KEYS, class EMIT, bool HINT = false, bool MARK = false>
__device__ __forceinline__ uint32_t select_row(TkShared& sh, int ncols, int k, KEYS keys, EMIT emit,
                                               uint32_t k2, uint32_t& thr_mask, uint32_t& thr_val,
                                               uint32_t hint_min = 0u, uint32_t hint_max = 0u,
                                               int nit = TK_ITEMS) {
    static_assert(!HINT || NSW == 1, "a range hint is for keys held in registers");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nsweep = NSW ? NSW : (ncols + TK_SWEEP - 1) / TK_SWEEP;
    uint32_t u[TK_ITEMS];
#pragma unroll
    for (int i = 0; i < TK_ITEMS; ++i) u[i] = 0u;
    // the bin list of a previous selection was last read before that
    // selection's final scan; the first barrier below orders this clear
    // before any append
    if (threadIdx.x == 0) sh.lcnt = 0u;

    // ---- count, min and max of the present keys; clear the histogram
    uint32_t n_present = 0xFFFFFFFFu, umin = hint_min, umax = hint_max;
    if (HINT) {
        keys(0, u);
    } else {
        uint32_t cnt = 0;
        umin = 0xFFFFFFFFu;
        umax = 0u;
        for (int s = 0; s < nsweep; ++s) {
            keys(s, u);
#pragma unroll
            for (int i = 0; i < TK_ITEMS; ++i) {
                if (i >= nit) break;
                if (u[i]) { cnt++; umin = min(umin, u[i]); umax = max(umax, u[i]); }
            }
        }
        for (int i = threadIdx.x; i < TK_BINS; i += TK_THREADS) sh.hist[i] = 0u;
        cnt = __builtin_amdgcn_readlane(wave_incl_sum(cnt), 63);
        umin = wave_min(umin);
        umax = wave_max(umax);
        if (lane == 0) { sh.red[0][wave] = cnt; sh.red[1][wave] = umin; sh.red[2][wave] = umax; }
        __syncthreads();
        n_present = 0;
        umin = 0xFFFFFFFFu; umax = 0u;
#pragma unroll
        for (int w = 0; w < TK_WAVES; ++w) {
            n_present += sh.red[0][w];
            umin = min(umin, sh.red[1][w]);
            umax = max(umax, sh.red[2][w]);
        }
    }

    // ---- radix select: prefix/mask describe the bits decided so far
    uint32_t prefix = 0u, mask = 0u, need = 0u;   // select (u & mask) > prefix, or == prefix for the first `need`
    int pb = 0;                                    // part buffer of the next scan
    thr_mask = 0u;
    thr_val = 0u;
    if (n_present > (uint32_t)k) {
        const uint32_t diff = umin ^ umax;
        int hb = diff ? 31 - __clz(diff) : -1;     // highest bit that is not common to all keys
        mask = hb < 0 ? 0xFFFFFFFFu : (hb >= 31 ? 0u : ~((2u << hb) - 1u));
        prefix = umin & mask;
        uint32_t rem = (uint32_t)k;
        uint32_t in_bin = n_present;
        int pass = 0;
        while (hb >= 0 && in_bin != rem) {
            if (in_bin <= 64u) {
                // At most 64 keys remain in the bin of the k-th key: list them
                // and let every wave rank them itself by (key descending,
                // column ascending), one list entry per lane.  The rem-th of
                // them is the threshold key T; the selection is then the keys
                // above T and the first rem' keys equal to T in column order,
                // which is what the final scan takes with mask = all bits.
                for (int s = 0; s < nsweep; ++s) {
                    if (nsweep > 1) keys(s, u);
                    const int c0 = s * TK_SWEEP + threadIdx.x * TK_ITEMS;
#pragma unroll
                    for (int i = 0; i < TK_ITEMS; ++i) {
                        if (i >= nit) break;
                        if (u[i] != 0u && (u[i] & mask) == prefix) {
                            const uint32_t slot = atomicAdd(&sh.lcnt, 1u);
                            sh.lkey[slot] = u[i];
                            sh.lcol[slot] = c0 + i;
                        }
                    }
                }
                __syncthreads();
                const uint32_t nl = __builtin_amdgcn_readfirstlane(in_bin);
                const bool has = (uint32_t)lane < nl;
                const uint32_t kj = has ? sh.lkey[lane] : 0u;
                const int cj = has ? sh.lcol[lane] : 0;
                uint32_t rank = 0u;
                for (uint32_t e = 0; e < nl; ++e) {
                    const uint32_t ke = __builtin_amdgcn_readlane(kj, e);
                    const int ce = __builtin_amdgcn_readlane(cj, e);
                    rank += (ke > kj) || (ke == kj && ce < cj);
                }
                // exactly one listed key has rank rem - 1 (1 <= rem <= nl)
                const uint64_t at = __ballot(has && rank == rem - 1u);
                const uint32_t t = __builtin_amdgcn_readlane(kj, (int)__builtin_ctzll(at));
                rem = (uint32_t)__popcll(__ballot(has && kj == t && rank < rem));
                prefix = t;
                mask = 0xFFFFFFFFu;
                break;
            }
            const int wbits = pass == 0 ? 12 : 10;
            const int shift = hb >= wbits - 1 ? hb - (wbits - 1) : 0;
            const int width = hb - shift + 1;
            const uint32_t dmask = (1u << width) - 1u;
            for (int s = 0; s < nsweep; ++s) {
                if (nsweep > 1) keys(s, u);
#pragma unroll
                for (int i = 0; i < TK_ITEMS; ++i) {
                    if (i >= nit) break;
                    if (u[i] != 0u && (u[i] & mask) == prefix) atomicAdd(&sh.hist[(u[i] >> shift) & dmask], 1u);
                }
            }
            __syncthreads();
            // thread t owns the 4 bins 4095-4t .. 4092-4t (descending digits);
            // it reads them once and clears them for the next pass
            const int b0 = TK_BINS - 4 - 4 * threadIdx.x;
            const uint4 hv = *(const uint4*)&sh.hist[b0];
            *(uint4*)&sh.hist[b0] = make_uint4(0u, 0u, 0u, 0u);
            const uint32_t hb4[4] = {hv.w, hv.z, hv.y, hv.x};
            const uint32_t h = hb4[0] + hb4[1] + hb4[2] + hb4[3];
            uint32_t tot;
            uint32_t before = block_excl_scan(h, sh.part[pb], tot);
            pb ^= 1;
            if (HINT && pass == 0 && tot <= rem) {
                // at most k present keys: every one is taken
                mask = 0u;
                prefix = 0u;
                break;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (hb4[j] != 0u && before < rem && rem <= before + hb4[j]) {
                    sh.digit = (uint32_t)(b0 + 3 - j);
                    sh.above = before;
                    sh.count = hb4[j];
                }
                // first pass: every present key is in the histogram, rem == k
                if (pass == 0 && hb4[j] != 0u && before < k2 && k2 <= before + hb4[j]) sh.digit2 = (uint32_t)(b0 + 3 - j);
                before += hb4[j];
            }
            __syncthreads();
            if (pass == 0 && k2 > 0u && k2 < (uint32_t)k) {
                thr_mask = mask | (dmask << shift);
                thr_val = prefix | (sh.digit2 << shift);
            }
            prefix |= sh.digit << shift;
            mask |= dmask << shift;
            rem -= sh.above;
            in_bin = sh.count;
            hb = shift - 1;
            ++pass;
        }
        need = rem;
    } else {
        need = (uint32_t)k;        // mask = prefix = 0: every present key counts as equal and is taken
    }

    // ---- selection in column order: one scan of (greater, equal) counts; the
    // equal items taken before a thread are min(equal before it, need).  The
    // thread's selected items are a 16-bit mask, emitted by walking its set
    // bits (a few per thread), not by a pass over all 16 items.
    uint32_t gt_base = 0u, eq_base = 0u;
    for (int s = 0; s < nsweep; ++s) {
        if (nsweep > 1) keys(s, u);
        uint32_t gtm = 0u, eqm = 0u, mkm = 0u;
#pragma unroll
        for (int i = 0; i < TK_ITEMS; ++i) {
            if (i >= nit) break;
            const uint32_t hi = u[i] & mask;
            gtm |= (uint32_t)(u[i] != 0u && hi > prefix) << i;
            eqm |= (uint32_t)(u[i] != 0u && hi == prefix) << i;
            if (MARK) mkm |= (uint32_t)((u[i] & thr_mask) >= thr_val) << i;
        }
        uint32_t tot;
        const uint32_t ex = block_excl_scan(((uint32_t)__builtin_popcount(gtm) << 16) | (uint32_t)__builtin_popcount(eqm),
                                            sh.part[pb], tot);
        pb ^= 1;
        const uint32_t eq_before = eq_base + (ex & 0xFFFFu);
        uint32_t pos = gt_base + (ex >> 16) + min(eq_before, need);
        // equal items: the first need - eq_before of this thread's, in column order
        uint32_t selm = gtm;
        for (uint32_t take = need > eq_before ? need - eq_before : 0u; eqm != 0u && take != 0u; --take) {
            selm |= eqm & (0u - eqm);
            eqm &= eqm - 1u;
        }
        const int c0 = s * TK_SWEEP + threadIdx.x * TK_ITEMS;
        while (selm != 0u) {
            const int i = __builtin_ctz(selm);
            selm &= selm - 1u;
            emit(c0 + i, pos, (mkm >> i) & 1u);
            ++pos;
        }
        gt_base += tot >> 16;
        eq_base += tot & 0xFFFFu;
    }
    return gt_base + min(eq_base, need);
}

// The first radix pass alone, over N keys per thread held in registers
// (0 = absent): (thr_mask, thr_val) such that the keys with
// (u & thr_mask) >= thr_val are the k largest and the other keys of the
// histogram bin that holds the k-th largest (every present key when there
// are at most k), and the largest key.  Leaves the histogram cleared.
template <int N>
__device__ __forceinline__ void kth_bin(TkShared& sh, const uint32_t* u, uint32_t k, uint32_t& thr_mask,
                                        uint32_t& thr_val, uint32_t& key_max) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t cnt = 0, umin = 0xFFFFFFFFu, umax = 0u;
#pragma unroll
    for (int i = 0; i < N; ++i)
        if (u[i]) { cnt++; umin = min(umin, u[i]); umax = max(umax, u[i]); }
    for (int i = threadIdx.x; i < TK_BINS; i += TK_THREADS) sh.hist[i] = 0u;
    cnt = __builtin_amdgcn_readlane(wave_incl_sum(cnt), 63);
    umin = wave_min(umin);
    umax = wave_max(umax);
    if (lane == 0) { sh.red[0][wave] = cnt; sh.red[1][wave] = umin; sh.red[2][wave] = umax; }
    __syncthreads();
    uint32_t n_present = 0;
    umin = 0xFFFFFFFFu; umax = 0u;
#pragma unroll
    for (int w = 0; w < TK_WAVES; ++w) {
        n_present += sh.red[0][w];
        umin = min(umin, sh.red[1][w]);
        umax = max(umax, sh.red[2][w]);
    }
    key_max = umax;
    thr_mask = 0u;
    thr_val = 0u;
    const uint32_t diff = umin ^ umax;
    if (n_present <= k || !diff) return;          // every present key (all of them equal in the second case)
    const int hb = 31 - __clz(diff);
    const uint32_t mask = hb >= 31 ? 0u : ~((2u << hb) - 1u);
    const uint32_t prefix = umin & mask;
    const int shift = hb >= 11 ? hb - 11 : 0;
    const uint32_t dmask = (1u << (hb - shift + 1)) - 1u;
#pragma unroll
    for (int i = 0; i < N; ++i)
        if (u[i] != 0u) atomicAdd(&sh.hist[(u[i] >> shift) & dmask], 1u);
    __syncthreads();
    const int b0 = TK_BINS - 4 - 4 * threadIdx.x;
    const uint4 hv = *(const uint4*)&sh.hist[b0];
    *(uint4*)&sh.hist[b0] = make_uint4(0u, 0u, 0u, 0u);
    const uint32_t hb4[4] = {hv.w, hv.z, hv.y, hv.x};
    uint32_t tot;
    uint32_t before = block_excl_scan(hb4[0] + hb4[1] + hb4[2] + hb4[3], sh.part[0], tot);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (hb4[j] != 0u && before < k && k <= before + hb4[j]) sh.digit = (uint32_t)(b0 + 3 - j);
        before += hb4[j];
    }
    __syncthreads();
    thr_mask = mask | (dmask << shift);
    thr_val = prefix | (sh.digit << shift);
}

// Keys of 16 consecutive columns c0 .. c0+15 of a row (absent past ncols).
__device__ __forceinline__ void load_cols(const float* krow, int ncols, int c0, uint32_t* u) {
    if (c0 + TK_ITEMS <= ncols && ((uintptr_t)(krow + c0) & 15) == 0) {
#pragma unroll
        for (int i = 0; i < TK_ITEMS; i += 4) {
            const float4 v = *(const float4*)(krow + c0 + i);
            u[i] = order_key(v.x); u[i + 1] = order_key(v.y); u[i + 2] = order_key(v.z); u[i + 3] = order_key(v.w);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < TK_ITEMS; ++i) {
        const int c = c0 + i;
        u[i] = c < ncols ? order_key(krow[c]) : 0u;
    }
}

// Keys of the two pool blocks behind columns c0 .. c0+15 (c0 a multiple of
// 16), read by position from a 16-B aligned row: two runs of 8 keys.  A
// negative pool entry marks a block that is skipped (its keys are absent).
__device__ __forceinline__ void load_pool_keys(const float* krow, const int32_t* pool, int ncols, int c0, uint32_t* u) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int cb = c0 + 8 * h;
        if (cb < ncols && pool[cb >> 3] >= 0) {
            const float* p = krow + 8 * pool[cb >> 3];
            const float4 v0 = *(const float4*)p, v1 = *(const float4*)(p + 4);
            const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) u[8 * h + i] = cb + i < ncols ? order_key(v[i]) : 0u;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) u[8 * h + i] = 0u;
        }
    }
}

// Keys of the 8 blocks of super-block sb (blocks 8 sb .. 8 sb + 7; absent
// past nb or for sb < 0): two 16-B loads where the run is whole and aligned.
__device__ __forceinline__ void load_block8(const float* brow, int nb, int sb, uint32_t* u) {
    const float* p = brow + 8 * (int64_t)(sb >= 0 ? sb : 0);
    if (sb >= 0 && 8 * sb + 8 <= nb && ((uintptr_t)p & 15) == 0) {
        const float4 v0 = *(const float4*)p, v1 = *(const float4*)(p + 4);
        u[0] = order_key(v0.x); u[1] = order_key(v0.y); u[2] = order_key(v0.z); u[3] = order_key(v0.w);
        u[4] = order_key(v1.x); u[5] = order_key(v1.y); u[6] = order_key(v1.z); u[7] = order_key(v1.w);
        return;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] = (sb >= 0 && 8 * sb + i < nb) ? order_key(p[i]) : 0u;
}

// x0 for columns 0..7 of a thread's 16, x1 for columns 8..15: a bitwise
// select (a ternary on the column, inside the loop over selected items, is
// turned into a two-entry table in scratch memory)
__device__ __forceinline__ int pick8(int col, int x0, int x1) {
    const int m = -((col >> 3) & 1);
    return (x0 & ~m) | (x1 & m);
}

__device__ __forceinline__ int col_id(const int32_t* pool, int c) {
    return pool ? 8 * pool[c >> 3] + (c & 7) : c;
}

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(TopkArgs a) {
    __shared__ TkShared sh;
    const int row = blockIdx.x;
    int ncols = a.max_cols;
    if (a.n_cols) {
        const int64_t v = ((int64_t)a.n_cols[row] * a.cols_mul + a.cols_div - 1) / a.cols_div;
        ncols = (int)(v < a.max_cols ? (v > 0 ? v : 0) : a.max_cols);
    }
    const float* krow = a.keys + (int64_t)row * a.key_stride;
    const int32_t* pool = a.pool ? a.pool + (int64_t)row * a.pool_stride : nullptr;
    int32_t* orow = a.out_ids + (int64_t)row * a.out_stride;
    auto keys = [&](int s, uint32_t* u) {
        const int c0 = s * TK_SWEEP + threadIdx.x * TK_ITEMS;
        if (a.keys_by_id) load_pool_keys(krow, pool, ncols, c0, u);
        else load_cols(krow, ncols, c0, u);
    };
    // selected columns are staged in LDS (the histogram is free once the
    // threshold is known) and leave in coalesced runs
    auto emit = [&](int col, uint32_t slot, uint32_t) { sh.hist[slot] = (uint32_t)col; };
    uint32_t thr_mask, thr_val;
    uint32_t n;
    if (ncols <= TK_SWEEP) {
        // Keys held in registers.  The k largest keys are at least the k-th
        // largest maximum of any partition of the row into groups (those k
        // maxima are k distinct keys), so one radix pass over the maxima of
        // each thread's two groups of 8 columns bounds them from below: keys
        // under that pass's bin of the k-th largest maximum are dropped, and
        // the selection proper runs over the rest (the same result, ties
        // included, with far fewer histogram atomics).
        uint32_t u[TK_ITEMS];
        keys(0, u);
        uint32_t gm[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < TK_ITEMS; ++i) gm[i >> 3] = max(gm[i >> 3], u[i]);
        uint32_t fmask, fval, kmax;
        kth_bin<2>(sh, gm, (uint32_t)a.k, fmask, fval, kmax);
        auto cand = [&](int, uint32_t* v) {
#pragma unroll
            for (int i = 0; i < TK_ITEMS; ++i) v[i] = (u[i] & fmask) >= fval ? u[i] : 0u;
        };
        n = select_row<1, decltype(cand), decltype(emit), true>(sh, ncols, a.k, cand, emit, 0u, thr_mask,
                                                                thr_val, fval, kmax);
    } else {
        n = select_row<0>(sh, ncols, a.k, keys, emit, 0u, thr_mask, thr_val);
    }
    __syncthreads();
    const int32_t* irow = a.ids ? a.ids + (int64_t)row * a.ids_stride : nullptr;
    for (int j = threadIdx.x; j < a.k; j += TK_THREADS)
        orow[j] = j < (int)n ? (irow ? irow[sh.hist[j]] : col_id(pool, (int)sh.hist[j])) : -1;
    if (threadIdx.x == 0) a.out_count[row] = (int32_t)n;
}

// The Full layer's selection for one row: the pool (top n_pool blocks by
// block maximum) and then the top k positions among the pool's scores.
//
// With a grid of two workgroups per row (rows of at most 16,384 blocks,
// k <= n_pool) the two results are computed side by side: workgroup y = 0
// selects the pool; y = 1 selects the positions without waiting for it.
// The top k positions lie in the top k blocks (below), hence in the pool and
// among the blocks whose maximum reaches the histogram bin of the k-th largest
// block maximum; y = 1 gathers the scores of those blocks only (if there are
// more than the pool size, of the top k blocks) and selects among them.
//
// PATH (chosen by the launcher, one instantiation each so that the register
// allocation of one form does not weigh on the others): SF_SPLIT, two
// workgroups per row; SF_REG, one per row, every row of at most 16,384 x 8
// blocks (held in registers); SF_ANY, one per row, any length.
constexpr int SF_SPLIT = 0, SF_REG = 1, SF_ANY = 2;

// the select kernel's LDS: the top-k state and the row's super-block maxima
struct __align__(16) SfShared : TkShared {
    uint32_t sbk[TK_SWEEP];            // order key of the maximum of each super-block of 8 blocks
};

template <int PATH>
__global__ __launch_bounds__(TK_THREADS) void select_full_kernel(SelectFullArgs a) {
    __shared__ SfShared sh;
    const int row = blockIdx.x;
    constexpr bool split = PATH == SF_SPLIT;
    const int nv = max(0, min(a.n_vis[row], a.max_vis));
    const int nb = (nv + 7) >> 3;
    const float* brow = a.block_max + (int64_t)row * a.block_max_stride;
    const float* srow = a.scores + (int64_t)row * a.scores_stride;
    int32_t* prow = a.pool + (int64_t)row * a.pool_stride;
    int32_t* irow = a.idx + (int64_t)row * a.idx_stride;

    // ---- blocks.  The top k positions lie in the top k blocks: a block ranked
    // above the block of a top-k position holds a distinct position ranked
    // above that position (its maximum; on equal values its lower id), so
    // fewer than k blocks rank above it.  The first radix pass bounds the top
    // k blocks from below by a histogram bin; pool blocks below that bin are
    // kept in the pool but marked (negative in LDS) and not read again.
    uint32_t thr_mask = 0u, thr_val = 0u;
    auto bkeys = [&](int s, uint32_t* u) { load_cols(brow, nb, s * TK_SWEEP + threadIdx.x * TK_ITEMS, u); };
    auto bemit = [&](int col, uint32_t slot, uint32_t mark) {
        sh.pool[slot] = mark ? col : (int32_t)((uint32_t)col | 0x80000000u);
    };
    if (!split && nb <= a.n_pool && nv <= TK_SWEEP) {
        // Every block is in the pool (blocks 0 .. nb-1, ascending; block
        // maxima of visible blocks are finite), so the top k positions are
        // the top k of the whole row: taken directly among its scores, held
        // in registers, after the group-maximum bound of the k-th key (the
        // groups of 8 columns are the blocks).  Same ids as the pool route.
        for (int j = threadIdx.x; j < a.n_pool; j += TK_THREADS) prow[j] = j < nb ? j : -1;
        if (threadIdx.x == 0) a.pool_count[row] = nb;
        uint32_t u[TK_ITEMS];
        load_cols(srow, nv, TK_ITEMS * (int)threadIdx.x, u);
        uint32_t gm[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < TK_ITEMS; ++i) gm[i >> 3] = max(gm[i >> 3], u[i]);
        uint32_t fmask, fval, kmax;
        kth_bin<2>(sh, gm, (uint32_t)a.k, fmask, fval, kmax);
        auto dkeys = [&](int, uint32_t* v) {
#pragma unroll
            for (int i = 0; i < TK_ITEMS; ++i) v[i] = (u[i] & fmask) >= fval ? u[i] : 0u;
        };
        auto demit = [&](int col, uint32_t slot, uint32_t) { sh.hist[slot] = (uint32_t)col; };
        uint32_t m3, v3;
        const uint32_t nd = select_row<1, decltype(dkeys), decltype(demit), true>(sh, nv, a.k, dkeys, demit, 0u, m3,
                                                                                  v3, fval, kmax);
        __syncthreads();
        for (int j = threadIdx.x; j < a.k; j += TK_THREADS) irow[j] = j < (int)nd ? (int32_t)sh.hist[j] : -1;
        if (threadIdx.x == 0) a.idx_count[row] = (int32_t)nd;
        return;
    }
    uint32_t np;
    if (split && blockIdx.y == 0) {
        // the pool alone, emitted straight into the output row
        auto pemit0 = [&](int col, uint32_t slot, uint32_t) { prow[slot] = col; };
        uint32_t m, v;
        np = select_row<1>(sh, nb, a.n_pool, bkeys, pemit0, 0u, m, v);
        for (int j = (int)np + threadIdx.x; j < a.n_pool; j += TK_THREADS) prow[j] = -1;
        if (threadIdx.x == 0) a.pool_count[row] = (int32_t)np;
        return;
    } else if (split && nv <= TK_SWEEP) {
        // a short row: its top k positions directly, among all its scores
        auto skeys2 = [&](int, uint32_t* uu) { load_cols(srow, nv, TK_ITEMS * (int)threadIdx.x, uu); };
        auto semit2 = [&](int col, uint32_t s2, uint32_t) { irow[s2] = col; };
        uint32_t m2, v2;
        const uint32_t ni = select_row<1>(sh, nv, a.k, skeys2, semit2, 0u, m2, v2);
        for (int j = (int)ni + threadIdx.x; j < a.k; j += TK_THREADS) irow[j] = -1;
        if (threadIdx.x == 0) a.idx_count[row] = (int32_t)ni;
        return;
    } else if (split) {
        // Candidate blocks: those at or above the histogram bin of the k-th
        // largest maximum of the super-blocks of 8 blocks (the k largest
        // super-block maxima are k distinct block maxima, so that bin's lower
        // edge bounds the k-th block maximum from below; the radix pass runs
        // over 2 keys per thread instead of 16).
        // Wave w holds blocks 1024 w .. 1024 w + 1023; it lists its candidates
        // (ascending) in sh.pool[128 w ..] with a wave-level prefix sum and
        // lane j gathers the scores of list entry j (a list of at most 64) or
        // of entries 2j and 2j + 1, so
        // thread order then item order is position order and no workgroup-wide
        // step is needed before the positions' selection.  A wave with more
        // than 128 candidates (ties) raises its flag; the selection is then
        // redone from the top k blocks.
        uint32_t u[TK_ITEMS];
        bkeys(0, u);
        uint32_t sbk[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i) { sbk[0] = max(sbk[0], u[i]); sbk[1] = max(sbk[1], u[8 + i]); }
        uint32_t key_max;
        kth_bin<2>(sh, sbk, (uint32_t)a.k, thr_mask, thr_val, key_max);
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        uint32_t flags = 0u, c = 0u;
#pragma unroll
        for (int i = 0; i < TK_ITEMS; ++i) {
            const bool cand = u[i] != 0u && (u[i] & thr_mask) >= thr_val;
            flags |= (uint32_t)cand << i;
            c += cand;
        }
        const uint32_t incl = wave_incl_sum(c);
        const uint32_t wtot = __builtin_amdgcn_readlane(incl, 63);
        int32_t* wlist = sh.pool + 128 * wave;
        uint32_t slot = incl - c;
#pragma unroll
        for (int i = 0; i < TK_ITEMS; ++i) {
            if (((flags >> i) & 1u) && slot < 128u) wlist[slot] = TK_ITEMS * (int)threadIdx.x + i;
            slot += (flags >> i) & 1u;
        }
        if (lane == 0) sh.ovf[wave] = wtot > 128u;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // at most 64 candidates: one block per lane (items 0..7, the passes
        // below stop after item 7); else two
        const bool one = wtot <= 64u;
        const int nit = one ? 8 : TK_ITEMS;
        const int e0 = one ? lane : 2 * lane;
        const int cb0 = e0 < (int)wtot ? wlist[e0] : -1;
        const int cb1 = !one && e0 + 1 < (int)wtot ? wlist[e0 + 1] : -1;
        uint32_t v[TK_ITEMS];
#pragma unroll
        for (int i = 8; i < TK_ITEMS; ++i) v[i] = 0u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (h && one) break;
            const int cb = h ? cb1 : cb0;
            const float4* p = (const float4*)(srow + 8 * (cb >= 0 ? cb : 0));
            const float4 v0 = p[0], v1 = p[1];
            const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t key = cb >= 0 && 8 * cb + i < nv ? order_key(f[i]) : 0u;
                v[8 * h + i] = (key & thr_mask) >= thr_val ? key : 0u;
            }
        }
        auto rkeys = [&](int, uint32_t* uu) {
#pragma unroll
            for (int i = 0; i < TK_ITEMS; ++i) uu[i] = v[i];
        };
        // positions go straight to the output row (the fallback below rewrites
        // every slot of it)
        auto remit = [&](int col, uint32_t s2, uint32_t) { irow[s2] = 8 * pick8(col, cb0, cb1) + (col & 7); };
        // every present key lies in [thr_val, key_max] (no score exceeds the
        // largest block maximum) and kth_bin left the histogram clear
        uint32_t m2, v2;
        const uint32_t ni = select_row<1, decltype(rkeys), decltype(remit), true>(sh, TK_SWEEP, a.k, rkeys, remit, 0u,
                                                                               m2, v2, thr_val, key_max, nit);
        // the flags were written before the selection's first barrier (its
        // first pass's)
        bool ovf_any = false;
#pragma unroll
        for (int w = 0; w < TK_WAVES; ++w) ovf_any |= sh.ovf[w] != 0u;
        if (!ovf_any) {
            for (int j = (int)ni + threadIdx.x; j < a.k; j += TK_THREADS) irow[j] = -1;
            if (threadIdx.x == 0) a.idx_count[row] = (int32_t)ni;
            return;
        }
        __syncthreads();
        auto temit = [&](int col, uint32_t s2, uint32_t) { sh.pool[s2] = col; };
        uint32_t m, vv;
        np = select_row<1>(sh, nb, a.k, bkeys, temit, 0u, m, vv);
    } else if (nb <= TK_SWEEP) {
        np = select_row<1, decltype(bkeys), decltype(bemit), false, true>(sh, nb, a.n_pool, bkeys, bemit, (uint32_t)a.k,
                                                                         thr_mask, thr_val);
    } else if (PATH == SF_REG || nb <= 8 * TK_SWEEP) {
        // Longer rows, in registers: the top n_pool blocks lie in the top
        // n_pool super-blocks of 8 blocks ranked by their maximum (a super-
        // block ranked above the one of a top block holds a distinct block
        // ranked above it: its maximum, on equal values with a lower id).
        // The super-block maxima are formed once, into LDS, from loads in
        // which consecutive threads read consecutive super-blocks (a wave's
        // load covers 2 KB of the row), 4 super-blocks per thread in flight;
        // the selection then reads thread t's super-blocks 16t .. 16t+15
        // from LDS.
        const int nsb = (nb + 7) >> 3;
#pragma unroll 1
        for (int j0 = 0; j0 * TK_THREADS < nsb; j0 += 4) {
            uint32_t b[4][8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int sb = (j0 + j) * TK_THREADS + (int)threadIdx.x;
                load_block8(brow, nb, sb < nsb ? sb : -1, b[j]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int sb = (j0 + j) * TK_THREADS + (int)threadIdx.x;
                uint32_t m = 0u;
#pragma unroll
                for (int i = 0; i < 8; ++i) m = max(m, b[j][i]);
                if (sb < nsb) sh.sbk[sb] = m;
            }
        }
        __syncthreads();
        auto skeys = [&](int, uint32_t* u) {
            const int c0 = TK_ITEMS * (int)threadIdx.x;
#pragma unroll
            for (int i = 0; i < TK_ITEMS; i += 4) {
                const uint4 v = *(const uint4*)&sh.sbk[c0 + i];   // c0 + 15 < 16,384: in the array
                u[i] = c0 + i < nsb ? v.x : 0u;
                u[i + 1] = c0 + i + 1 < nsb ? v.y : 0u;
                u[i + 2] = c0 + i + 2 < nsb ? v.z : 0u;
                u[i + 3] = c0 + i + 3 < nsb ? v.w : 0u;
            }
        };
        auto semit = [&](int col, uint32_t slot, uint32_t) { sh.pool[slot] = col; };
        uint32_t s_mask, s_val;
        const uint32_t nsp = select_row<1>(sh, nsb, a.n_pool, skeys, semit, 0u, s_mask, s_val);
        __syncthreads();                              // the chosen super-blocks, ascending, are in sh.pool
        // candidate column c is block 8 * super[c / 8] + c % 8; thread t's
        // columns belong to super-blocks 2t and 2t + 1 of the list (read here,
        // before the selection below rewrites sh.pool at its end)
        const int sb0 = 2 * (int)threadIdx.x < (int)nsp ? sh.pool[2 * threadIdx.x] : -1;
        const int sb1 = 2 * (int)threadIdx.x + 1 < (int)nsp ? sh.pool[2 * threadIdx.x + 1] : -1;
        auto ckeys = [&](int, uint32_t* u) {
            load_block8(brow, nb, sb0, u);
            load_block8(brow, nb, sb1, u + 8);
        };
        auto cemit = [&](int col, uint32_t slot, uint32_t mark) {
            const int blk = 8 * pick8(col, sb0, sb1) + (col & 7);
            sh.pool[slot] = mark ? blk : (int32_t)((uint32_t)blk | 0x80000000u);
        };
        np = select_row<1, decltype(ckeys), decltype(cemit), false, true>(sh, 8 * (int)nsp, a.n_pool, ckeys, cemit,
                                                                         (uint32_t)a.k, thr_mask, thr_val);
    } else {
        np = select_row<0, decltype(bkeys), decltype(bemit), false, true>(sh, nb, a.n_pool, bkeys, bemit, (uint32_t)a.k,
                                                                         thr_mask, thr_val);
    }
    __syncthreads();                                  // the pool is complete in LDS

    // ---- positions: column c is position 8 * pool[c/8] + c%8 (-inf past n_vis)
    const int ncols = 8 * (int)np;
    // The k largest block maxima are k distinct scores, so the k-th largest
    // score is at least the k-th largest block maximum: positions below the
    // histogram bin of that block are dropped as they are read.
    auto pkeys = [&](int s, uint32_t* u) {
        load_pool_keys(srow, sh.pool, ncols, s * TK_SWEEP + threadIdx.x * TK_ITEMS, u);
#pragma unroll
        for (int i = 0; i < TK_ITEMS; ++i) u[i] = (u[i] & thr_mask) >= thr_val ? u[i] : 0u;
    };
    // Thread t's columns 16t .. 16t+15 are pool blocks 2t and 2t+1; only
    // candidate blocks have present keys, so the entries used are >= 0.
    const int pb0 = 2 * (int)threadIdx.x < (int)np ? 8 * (sh.pool[2 * threadIdx.x] & 0x7FFFFFFF) : 0;
    const int pb1 = 2 * (int)threadIdx.x + 1 < (int)np ? 8 * (sh.pool[2 * threadIdx.x + 1] & 0x7FFFFFFF) : 0;
    auto pemit = [&](int col, uint32_t slot, uint32_t) { sh.hist[slot] = (uint32_t)(pick8(col, pb0, pb1) + (col & 7)); };
    uint32_t thr2_mask, thr2_val;
    const uint32_t ni = select_row<1>(sh, ncols, a.k, pkeys, pemit, 0u, thr2_mask, thr2_val);
    __syncthreads();

    // ---- outputs, from LDS in coalesced runs (no barrier waits on these stores)
    if (!split) {
        for (int j = threadIdx.x; j < a.n_pool; j += TK_THREADS) prow[j] = j < (int)np ? (sh.pool[j] & 0x7FFFFFFF) : -1;
        if (threadIdx.x == 0) a.pool_count[row] = (int32_t)np;
    }
    for (int j = threadIdx.x; j < a.k; j += TK_THREADS) irow[j] = j < (int)ni ? (int32_t)sh.hist[j] : -1;
    if (threadIdx.x == 0) a.idx_count[row] = (int32_t)ni;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)a.n_rows), dim3(TK_THREADS), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_select_full(const SelectFullArgs& a, hipStream_t st) {
    // two workgroups per row while the doubled grid still fits the 256 CUs
    // once (a workgroup fills a CU), for rows of more than 8 k blocks (fewer
    // super-blocks than k would make every block a candidate) and k <= 1,024
    // (about k candidates share the 16 waves' lists of 128); larger launches,
    // shorter rows and larger k keep one workgroup per row
    const bool split = a.max_vis > 64 * a.k && a.max_vis <= 8 * TK_SWEEP && a.k <= a.n_pool && a.k <= 1024 &&
                       2 * a.n_rows <= 256;
    const dim3 grid((unsigned)a.n_rows, split ? 2u : 1u), block(TK_THREADS);
    if (split) hipLaunchKernelGGL(select_full_kernel<SF_SPLIT>, grid, block, 0, st, a);
    else if ((a.max_vis + 7) / 8 <= 8 * TK_SWEEP) hipLaunchKernelGGL(select_full_kernel<SF_REG>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(select_full_kernel<SF_ANY>, grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace csa2
