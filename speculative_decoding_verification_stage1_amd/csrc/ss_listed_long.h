// Listed tokens of rows whose prior or bias list is longer than LIST_SHORT
// (penalty histories up to SS_PRIOR_MAX entries, bias lists up to
// SS_BIAS_MAX): the same result as listed_row_wave - the exact processed
// logit of every token named by an active list entry, as merge keys, the
// row's best 128 - by one workgroup per row instead of one wave, with the
// sorting form of ss_stage2.h (listed_entry_key, listed_token_key) over
// up to LL_CAP entries in LDS.  The tokens' keys are then reduced to the
// best 128 with the register bitonic sorts and merges of Stage 2.
#pragma once

#include "ss_stage2.h"

namespace ssd {

constexpr int LL_THREADS = 256;
constexpr int LL_CAP = 8192;   // >= SS_PRIOR_MAX + SS_GAMMA_MAX + SS_BIAS_MAX
static_assert(SS_PRIOR_MAX + SS_GAMMA_MAX + SS_BIAS_MAX <= LL_CAP, "sort capacity");
static_assert(LL_CAP < (1 << 16), "entry positions fit the key's low 16 bits");

struct LongShared {
    uint64_t k[LL_CAP];
    uint64_t wl[S2_WAVES][2][WAVE];
};

// Ascending bitonic sort of k[0, n), n a power of two, by the workgroup.
__device__ __forceinline__ void ll_sort(uint64_t* k, int n) {
    const int tid = threadIdx.x;
    for (int size = 2; size <= n; size <<= 1)
        for (int j = size >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < n / 2; i += LL_THREADS) {
                const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
                const int hi = lo + j;
                const uint64_t a = k[lo], c = k[hi];
                if ((a > c) == ((lo & size) == 0)) {
                    k[lo] = c;
                    k[hi] = a;
                }
            }
            __syncthreads();
        }
}

template <int DT>
__global__ __launch_bounds__(LL_THREADS) void listed_long_kernel(Stage1Params P) {
    __shared__ LongShared sh;
    const int row = blockIdx.x;
    if (!row_used(P, row)) return;
    const int b = __builtin_amdgcn_readfirstlane(div_uniform(row, P.rows_per_req));
    const RowParams rp = row_params(P, b);
    const int np = rp.valid ? rp.n_prior : 0;
    const int nb = rp.valid ? rp.n_bias : 0;
    if (np <= LIST_SHORT && nb <= LIST_SHORT) return;   // block-uniform: ranked in the Stage-1 launch
    const int nh = draft_hist_len(P, rp.flags, row);
    const int n = np + nh + nb;
    int ns = 256;
    while (ns < n) ns <<= 1;
    const int tid = threadIdx.x;
    // 1. entry keys (entries that name no token sort last), sorted
    for (int i = tid; i < ns; i += LL_THREADS) sh.k[i] = i < n ? listed_entry_key(P, b, i, np, nh) : ~0ull;
    __syncthreads();
    ll_sort(sh.k, ns);
    // 2. each token's key, by the thread holding its first entry
    constexpr int PER = LL_CAP / LL_THREADS;
    uint64_t res[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int i = tid + q * LL_THREADS;
        res[q] = i < ns ? listed_token_key<DT>(P, rp, row, b, sh.k, ns, i, np, nh) : 0ull;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < PER; ++q)
        if (tid + q * LL_THREADS < ns) sh.k[tid + q * LL_THREADS] = res[q];
    __syncthreads();
    // 3. the best 128: each wave sorts its chunks of 128 and merges them;
    //    then the cross-wave tree
    const int wave = tid / WAVE;
    const int lane = lane_id();
    WL64 mine{0ull, 0ull};
    for (int c0 = wave * KMAX; c0 < ns; c0 += S2_WAVES * KMAX) {
        const WL64 l = wave_sort128(WL64{sh.k[c0 + lane], sh.k[c0 + lane + WAVE]});
        mine = c0 == wave * KMAX ? l : wave_merge(mine, l);
    }
    sh.wl[wave][0][lane] = mine.lo;
    sh.wl[wave][1][lane] = mine.hi;
    __syncthreads();
    auto wl = [&](int w) -> WL64 { return WL64{sh.wl[w][0][lane], sh.wl[w][1][lane]}; };
    if (wave == 1) {
        const WL64 z = wave_merge(wl(2), wl(3));
        sh.wl[2][0][lane] = z.lo;
        sh.wl[2][1][lane] = z.hi;
    }
    WL64 best{0ull, 0ull};
    if (wave == 0) best = wave_merge(mine, wl(1));
    __syncthreads();
    if (wave == 0) {
        best = wave_merge(best, wl(2));
        P.listed[(int64_t)row * KMAX + lane] = best.lo;
        P.listed[(int64_t)row * KMAX + lane + WAVE] = best.hi;
    }
}

}  // namespace ssd
