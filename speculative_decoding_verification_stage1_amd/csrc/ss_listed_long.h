// Listed tokens of rows whose prior or bias list is longer than LIST_SHORT
// (penalty histories up to SS_PRIOR_MAX entries, bias lists up to
// SS_BIAS_MAX): the same result as listed_row_wave - the exact processed
// logit of every token named by an active list entry, as merge keys, the
// row's best 128 - by one workgroup per row instead of one wave.
//
// The row's entries (prior entries, then the earlier drafts of a
// verification row, then bias entries) become keys id << 16 | position and
// are sorted in LDS, so the entries of one token lie together in list
// order.  The first entry of each token then walks its entries and applies
// the list arithmetic in the order of the logits-processing definition:
// the repetition map once per live prior entry, then each prior entry's
// frequency/presence subtraction, then each bias addition; a token's
// earlier drafts add to the count of its first live prior entry, or form
// one appended entry.  The tokens' keys are then reduced to the best 128
// with the register bitonic sorts and merges of Stage 2.
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
    const int64_t po = (int64_t)b * P.aux.prior_stride, bo = (int64_t)b * P.aux.bias_stride;
    // 1. entry keys (entries that name no token sort last)
    for (int i = tid; i < ns; i += LL_THREADS) {
        uint64_t key = ~0ull;
        if (i < n) {
            int id;
            bool ok;
            if (i < np) {
                id = gmem(P.aux.prior_ids)[po + i];
                ok = gmem(P.aux.prior_cnt)[po + i] >= 1;
            } else if (i < np + nh) {
                id = gmem(P.draft_ids)[(int64_t)b * (P.rows_per_req - 1) + (i - np)];
                ok = true;
            } else {
                id = gmem(P.aux.bias_ids)[bo + (i - np - nh)];
                ok = true;
            }
            if (ok && id >= 0 && id < P.V) key = ((uint64_t)(uint32_t)id << 16) | (uint64_t)i;
        }
        sh.k[i] = key;
    }
    __syncthreads();
    ll_sort(sh.k, ns);
    // 2. each token's processed logit, by the thread holding its first entry
    const bool grammar = (rp.flags & SS_GRAMMAR) != 0;
    const bool do_rep = (rp.flags & SS_REP) != 0;
    const bool do_fp = (rp.flags & SS_FREQPRES) != 0;
    const bool do_bias = (rp.flags & SS_BIAS) != 0;
    constexpr int PER = LL_CAP / LL_THREADS;
    uint64_t res[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        res[q] = 0ull;
        const int i = tid + q * LL_THREADS;
        if (i >= ns) continue;
        const uint64_t e = sh.k[i];
        if (e == ~0ull) continue;
        const uint32_t id = (uint32_t)(e >> 16);
        if (i > 0 && sh.k[i - 1] != ~0ull && (uint32_t)(sh.k[i - 1] >> 16) == id) continue;   // not the first
        int end = i + 1;
        while (end < ns && sh.k[end] != ~0ull && (uint32_t)(sh.k[end] >> 16) == id) ++end;
        int first_prior = -1, ndraft = 0;
        for (int t = i; t < end; ++t) {
            const int pos = (int)(sh.k[t] & 0xFFFFu);
            if (pos < np) {
                if (first_prior < 0) first_prior = pos;
            } else if (pos < np + nh) {
                ++ndraft;
            }
        }
        const bool appended = first_prior < 0 && ndraft > 0;
        float z;
        if (DT == SS_BF16) z = widen_bf16(((const uint16_t*)P.logits)[(int64_t)row * P.ld + id]);
        else z = ((const float*)P.logits)[(int64_t)row * P.ld + id];
        if (grammar && !((P.aux.bitmask[(int64_t)row * P.aux.bitmask_stride + (id >> 5)] >> (id & 31)) & 1u))
            z = bitsf(F32_NINF_BITS);
        if (do_rep) {
            for (int t = i; t < end; ++t)
                if ((int)(sh.k[t] & 0xFFFFu) < np) z = (z > 0.0f) ? z / rp.rep : z * rp.rep;
            if (appended) z = (z > 0.0f) ? z / rp.rep : z * rp.rep;
        }
        if (do_fp) {
            for (int t = i; t < end; ++t) {
                const int pos = (int)(sh.k[t] & 0xFFFFu);
                if (pos >= np) continue;
                const int c = gmem(P.aux.prior_cnt)[po + pos] + (pos == first_prior ? ndraft : 0);
                z = z - ((float)c * rp.freq + rp.pres);
            }
            if (appended) z = z - ((float)ndraft * rp.freq + rp.pres);
        }
        if (do_bias)
            for (int t = i; t < end; ++t) {
                const int pos = (int)(sh.k[t] & 0xFFFFu);
                if (pos >= np + nh) z = z + gmem(P.aux.bias_val)[bo + (pos - np - nh)];
            }
        res[q] = ((uint64_t)ord32(canon(z)) << 32) | (uint64_t)(0xFFFFFFFFu - id);
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
