// topk.hip -- K3: exact row-wise top-k (gfx950).
//
// Top-k selector of the lightning indexer ['DeepSeek-V4' paper page, section
// 2.3.1] and the block-pool step of the hierarchical sparse indexer (groups
// of 8 positions ranked by their maximum, up to 2,048 kept; V4.1-Flash
// architecture page).  Rank = (key descending, column ascending); columns
// are in id order, so ties go to the lower position / block.
//
// One 1024-thread workgroup per row.  Keys become order-preserving 32-bit
// integers; an MSB-first radix select (four 8-bit digit passes over an LDS
// histogram) finds the k-th key T and how many items equal to T are needed;
// a block-wide scan in column order then writes the selected ids ascending.
// Thread t owns columns [16t, 16t+16) of each 16,384-column sweep, so
// "column order" is "thread order, then item order".  A row of at most
// 16,384 columns stays in registers; longer rows are re-read per pass.
#include "csa2_device.h"
#include "csa2_launch.h"

namespace csa2 {

constexpr int TK_THREADS = 1024;
constexpr int TK_ITEMS = 16;
constexpr int TK_SWEEP = TK_THREADS * TK_ITEMS;
constexpr int TK_WAVES = TK_THREADS / 64;

struct TkShared {
    uint32_t hist[256];
    uint32_t part[TK_WAVES];
    uint32_t digit, above;
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

__device__ __forceinline__ int col_id(const TopkArgs& a, const int32_t* pool, int c) {
    return pool ? 8 * pool[c >> 3] + (c & 7) : c;
}

__device__ __forceinline__ void load_sweep(const TopkArgs& a, const float* krow, const int32_t* pool,
                                           int ncols, int sweep, uint32_t* u) {
    const int c0 = sweep * TK_SWEEP + threadIdx.x * TK_ITEMS;
#pragma unroll
    for (int i = 0; i < TK_ITEMS; ++i) {
        const int c = c0 + i;
        uint32_t key = 0u;
        if (c < ncols) key = order_key(krow[a.keys_by_id ? col_id(a, pool, c) : c]);
        u[i] = key;
    }
}

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(TopkArgs a) {
    __shared__ TkShared sh;
    const int row = blockIdx.x;
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
    if (nsweep >= 1) load_sweep(a, krow, pool, ncols, 0, u);
    else {
#pragma unroll
        for (int i = 0; i < TK_ITEMS; ++i) u[i] = 0u;
    }

    // number of present keys
    uint32_t present = 0;
    for (int s = 0; s < nsweep; ++s) {
        if (s > 0) load_sweep(a, krow, pool, ncols, s, u);
#pragma unroll
        for (int i = 0; i < TK_ITEMS; ++i) present += u[i] != 0u;
    }
    uint32_t n_present;
    block_excl_scan(present, sh.part, n_present);

    uint32_t T = 0u, need_eq = 0u;
    if (n_present > (uint32_t)a.k) {
        uint32_t prefix = 0u, mask = 0u, rem = (uint32_t)a.k;
        for (int shift = 24; shift >= 0; shift -= 8) {
            if (threadIdx.x < 256) sh.hist[threadIdx.x] = 0u;
            __syncthreads();
            for (int s = 0; s < nsweep; ++s) {
                if (nsweep > 1) load_sweep(a, krow, pool, ncols, s, u);
#pragma unroll
                for (int i = 0; i < TK_ITEMS; ++i)
                    if (u[i] != 0u && (u[i] & mask) == prefix) atomicAdd(&sh.hist[(u[i] >> shift) & 255u], 1u);
            }
            __syncthreads();
            // digits in descending order: thread t looks at digit 255 - t
            const uint32_t h = threadIdx.x < 256 ? sh.hist[255 - threadIdx.x] : 0u;
            uint32_t tot;
            const uint32_t before = block_excl_scan(h, sh.part, tot);
            if (threadIdx.x < 256 && before < rem && rem <= before + h) {
                sh.digit = 255u - threadIdx.x;
                sh.above = before;
            }
            __syncthreads();
            prefix |= sh.digit << shift;
            mask |= 0xFFu << shift;
            rem -= sh.above;
            __syncthreads();
        }
        T = prefix;
        need_eq = rem;
    }

    // selection in column order
    uint32_t eq_base = 0u, out_base = 0u;
    for (int s = 0; s < nsweep; ++s) {
        if (nsweep > 1) load_sweep(a, krow, pool, ncols, s, u);
        uint32_t n_eq = 0u;
#pragma unroll
        for (int i = 0; i < TK_ITEMS; ++i) n_eq += (T != 0u && u[i] == T);
        uint32_t eq_tot;
        uint32_t eq_rank = eq_base + block_excl_scan(n_eq, sh.part, eq_tot);
        uint32_t sel_mask = 0u, n_sel = 0u;
#pragma unroll
        for (int i = 0; i < TK_ITEMS; ++i) {
            bool sel = u[i] > T;
            if (T != 0u && u[i] == T) {
                sel = eq_rank < need_eq;
                eq_rank++;
            }
            if (sel) { sel_mask |= 1u << i; n_sel++; }
        }
        uint32_t sel_tot;
        uint32_t pos = out_base + block_excl_scan(n_sel, sh.part, sel_tot);
        const int c0 = s * TK_SWEEP + threadIdx.x * TK_ITEMS;
#pragma unroll
        for (int i = 0; i < TK_ITEMS; ++i)
            if (sel_mask & (1u << i)) orow[pos++] = col_id(a, pool, c0 + i);
        eq_base += eq_tot;
        out_base += sel_tot;
    }
    for (int j = (int)out_base + threadIdx.x; j < a.k; j += TK_THREADS) orow[j] = -1;
    if (threadIdx.x == 0) a.out_count[row] = (int32_t)out_base;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)a.n_rows), dim3(TK_THREADS), 0, st, a);
    return hipGetLastError();
}

}  // namespace csa2
