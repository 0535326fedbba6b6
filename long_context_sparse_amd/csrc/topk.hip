// topk.hip -- K3: exact row-wise top-k (gfx950).
//
// Top-k selector of the lightning indexer ['DeepSeek-V4' paper page, section
// 2.3.1] and the block-pool step of the hierarchical sparse indexer (groups
// of 8 positions ranked by their maximum, up to 2,048 kept; V4.1-Flash
// architecture page).  Rank = (key descending, column ascending); columns
// are in id order, so ties go to the lower position / block.
//
// One 1024-thread workgroup per row.  Keys become order-preserving 32-bit
// integers.  The bits above the highest bit in which the smallest and the
// largest present key differ are common to every key and are skipped; an
// MSB-first radix select then resolves 12, 10 and 10 bits per pass with an
// LDS histogram of 4,096 bins (scores of one row share few exponent values,
// so a digit that covers only exponent bits would send most atomics to one
// bin; 12 bits reach into the mantissa), and stops as soon as the bin
// holding the k-th key is taken whole.  A block-wide scan in column order
// writes the selected ids ascending.  Thread t owns columns [16t, 16t+16) of
// each 16,384-column sweep, so column order is thread order, then item order.
// Rows of at most 16,384 columns stay in registers; longer rows are re-read.
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

constexpr int TK_THREADS = 1024;
constexpr int TK_ITEMS = 16;
constexpr int TK_SWEEP = TK_THREADS * TK_ITEMS;
constexpr int TK_WAVES = TK_THREADS / 64;

constexpr int TK_BINS = 4096;

struct TkShared {
    uint32_t hist[TK_BINS];
    uint32_t part[TK_WAVES];
    uint32_t red[3][TK_WAVES];
    uint32_t digit, above, count;
};

// Exclusive scan of v over the workgroup in thread order; `total` gets the sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* part, uint32_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) part[wave] = x;
    __syncthreads();
    if (wave == 0) {
        uint32_t p = lane < TK_WAVES ? part[lane] : 0u;
#pragma unroll
        for (int d = 1; d < TK_WAVES; d <<= 1) {
            const uint32_t y = __shfl_up(p, d, 64);
            if (lane >= d) p += y;
        }
        if (lane < TK_WAVES) part[lane] = p;
    }
    __syncthreads();
    const uint32_t base = wave > 0 ? part[wave - 1] : 0u;
    total = part[TK_WAVES - 1];
    __syncthreads();
    return base + x - v;
}

__device__ __forceinline__ int col_id(const int32_t* pool, int c) {
    return pool ? 8 * pool[c >> 3] + (c & 7) : c;
}

__device__ __forceinline__ void load_sweep(const TopkArgs& a, const float* krow, const int32_t* pool,
                                           int ncols, int sweep, uint32_t* u) {
    const int c0 = sweep * TK_SWEEP + threadIdx.x * TK_ITEMS;   // a multiple of 16
    if (a.keys_by_id) {
        // columns c0 .. c0+15 are the two pool blocks c0/8 and c0/8 + 1: two runs of 8 keys
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int cb = c0 + 8 * h;
            if (cb < ncols) {
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
        return;
    }
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

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(TopkArgs a) {
    __shared__ TkShared sh;
    const int row = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int ncols = a.max_cols;
    if (a.n_cols) {
        const int64_t v = ((int64_t)a.n_cols[row] * a.cols_mul + a.cols_div - 1) / a.cols_div;
        ncols = (int)(v < a.max_cols ? (v > 0 ? v : 0) : a.max_cols);
    }
    const int nsweep = (ncols + TK_SWEEP - 1) / TK_SWEEP;
    const float* krow = a.keys + (int64_t)row * a.key_stride;
    const int32_t* pool = a.pool ? a.pool + (int64_t)row * a.pool_stride : nullptr;
    int32_t* orow = a.out_ids + (int64_t)row * a.out_stride;

    uint32_t u[TK_ITEMS];
#pragma unroll
    for (int i = 0; i < TK_ITEMS; ++i) u[i] = 0u;

    // ---- count, min and max of the present keys
    uint32_t cnt = 0, umin = 0xFFFFFFFFu, umax = 0u;
    for (int s = 0; s < nsweep; ++s) {
        load_sweep(a, krow, pool, ncols, s, u);
#pragma unroll
        for (int i = 0; i < TK_ITEMS; ++i)
            if (u[i]) { cnt++; umin = min(umin, u[i]); umax = max(umax, u[i]); }
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        cnt += __shfl_xor(cnt, d, 64);
        umin = min(umin, (uint32_t)__shfl_xor(umin, d, 64));
        umax = max(umax, (uint32_t)__shfl_xor(umax, d, 64));
    }
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

    // ---- radix select: prefix/mask describe the bits decided so far
    uint32_t prefix = 0u, mask = 0u, need = 0u;   // select (u & mask) > prefix, or == prefix for the first `need`
    if (n_present > (uint32_t)a.k) {
        const uint32_t diff = umin ^ umax;
        int hb = diff ? 31 - __clz(diff) : -1;   // highest bit that is not common to all keys
        mask = hb < 0 ? 0xFFFFFFFFu : (hb >= 31 ? 0u : ~((2u << hb) - 1u));
        prefix = umin & mask;
        uint32_t rem = (uint32_t)a.k;
        uint32_t in_bin = n_present;
        int pass = 0;
        while (hb >= 0 && in_bin != rem) {
            const int wbits = pass == 0 ? 12 : 10;
            const int shift = hb >= wbits - 1 ? hb - (wbits - 1) : 0;
            const int width = hb - shift + 1;
            const uint32_t dmask = (1u << width) - 1u;
            for (int i = threadIdx.x; i < TK_BINS; i += TK_THREADS) sh.hist[i] = 0u;
            __syncthreads();
            for (int s = 0; s < nsweep; ++s) {
                if (nsweep > 1) load_sweep(a, krow, pool, ncols, s, u);
#pragma unroll
                for (int i = 0; i < TK_ITEMS; ++i)
                    if (u[i] != 0u && (u[i] & mask) == prefix) atomicAdd(&sh.hist[(u[i] >> shift) & dmask], 1u);
            }
            __syncthreads();
            // thread t owns the 4 bins 4095-4t .. 4092-4t (descending digits)
            uint32_t hb4[4], h = 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) { hb4[j] = sh.hist[TK_BINS - 1 - 4 * threadIdx.x - j]; h += hb4[j]; }
            uint32_t tot;
            uint32_t before = block_excl_scan(h, sh.part, tot);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (hb4[j] != 0u && before < rem && rem <= before + hb4[j]) {
                    sh.digit = (uint32_t)(TK_BINS - 1 - 4 * threadIdx.x - j);
                    sh.above = before;
                    sh.count = hb4[j];
                }
                before += hb4[j];
            }
            __syncthreads();
            prefix |= sh.digit << shift;
            mask |= dmask << shift;
            rem -= sh.above;
            in_bin = sh.count;
            hb = shift - 1;
            ++pass;
            __syncthreads();
        }
        need = rem;
    }
    const bool take_all = n_present <= (uint32_t)a.k;

    // ---- selection in column order: one scan of (greater, equal) counts; the
    // equal items taken before a thread are min(equal before it, need)
    uint32_t gt_base = 0u, eq_base = 0u, out_base = 0u;
    for (int s = 0; s < nsweep; ++s) {
        if (nsweep > 1) load_sweep(a, krow, pool, ncols, s, u);
        uint32_t n_gt = 0u, n_eq = 0u;
#pragma unroll
        for (int i = 0; i < TK_ITEMS; ++i) {
            if (u[i] == 0u) continue;
            if (take_all) { n_gt++; continue; }
            const uint32_t hi = u[i] & mask;
            n_gt += hi > prefix;
            n_eq += hi == prefix;
        }
        uint32_t tot;
        const uint32_t ex = block_excl_scan((n_gt << 16) | n_eq, sh.part, tot);
        uint32_t eq_rank = eq_base + (ex & 0xFFFFu);
        uint32_t pos = gt_base + (ex >> 16) + min(eq_rank, need);
        const int c0 = s * TK_SWEEP + threadIdx.x * TK_ITEMS;
#pragma unroll
        for (int i = 0; i < TK_ITEMS; ++i) {
            if (u[i] == 0u) continue;
            bool sel;
            if (take_all) sel = true;
            else {
                const uint32_t hi = u[i] & mask;
                sel = hi > prefix;
                if (hi == prefix) { sel = eq_rank < need; eq_rank++; }
            }
            if (sel) orow[pos++] = col_id(pool, c0 + i);
        }
        gt_base += tot >> 16;
        eq_base += tot & 0xFFFFu;
    }
    out_base = gt_base + min(eq_base, need);
    for (int j = (int)out_base + threadIdx.x; j < a.k; j += TK_THREADS) orow[j] = -1;
    if (threadIdx.x == 0) a.out_count[row] = (int32_t)out_base;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)a.n_rows), dim3(TK_THREADS), 0, st, a);
    return hipGetLastError();
}

}  // namespace csa2
