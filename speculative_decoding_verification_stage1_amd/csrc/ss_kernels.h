// Kernel entry points.  A sampling step is two launches: Stage 1 over all
// (row, tile) pairs, then Stage 2 with one workgroup per row; verification
// adds one launch with one workgroup per request.  The kernel boundaries are
// the only synchronisation between workgroups (the Stage-1 keys cross in
// the workspace).
#pragma once

#include "ss_verify.h"

namespace ssd {

template <int DT>
union S1KernelShared {
    S1Shared<DT> tile;
    ListedArea lists[S1_WAVES];
};

// The first ceil(listed_rows / 4) workgroups compute the rows' listed
// tokens (ranked in Stage 2), one row per wave; the rest each own one
// (row, tile).  The listed workgroups come first so they run alongside the
// streaming, not after it.
template <int DT>
__global__ __launch_bounds__(S1_THREADS) void stage1_kernel(Stage1Params P) {
    using Key = typename S1Traits<DT>::Key;
    __shared__ S1KernelShared<DT> shu;
    const int tid = threadIdx.x;
    if (blockIdx.x == 0 && tid == 0 && P.rng_snap) {   // the step's copy of the generator state
        ss_rng r{0ull, 0ull};
        if (P.rng) r = *P.rng;
        *P.rng_snap = r;
        if (P.rng && P.rng_advance) P.rng->offset = r.offset + P.rng_advance;
    }
    // verification: the requests' decision words start at zero (Stage 2
    // adds to them with device-scope atomics after this launch has
    // completed; device-coherent stores, as for the rest of that hand-off)
    if (blockIdx.x == 0)
        for (int i = tid; i < P.n_clear; i += S1_THREADS) store_coherent(P.clear_words + i, (uint64_t)0);
    const int nlw = (P.listed_rows + S1_WAVES - 1) / S1_WAVES;
    if ((int)blockIdx.x < nlw) {
        const int wave = tid / WAVE;
        const int r = (int)blockIdx.x * S1_WAVES + wave;
        if (r < P.listed_rows && row_used(P, r)) listed_row_wave<DT>(P, P.listed, r, shu.lists[wave]);
        return;
    }
    S1Shared<DT>& sh = shu.tile;
    // the tile waves issue ahead of listed-token waves sharing their SIMDs
    // (those finish well before the tiles do, except the sorting form, which
    // raises its own priority above): 64 rows of 2^17 bf16, Stage 1 10.38 ->
    // 10.03 us; verification of 64 requests x 5 rows of 2^17, 29.44 ->
    // 29.18 us; 256 rows of 2^18 unchanged
    __builtin_amdgcn_s_setprio(1);
    const int wg = blockIdx.x - nlw;
    const int row = div_uniform(wg, P.Zv);
    const int tile = wg - row * P.Zv;
    if (!row_used(P, row)) return;   // no loads for a row past its request's bonus position
    WList<Key> res{0, 0};
    stage1_tile<DT>(P, row, tile, sh, &res);
    if (tid / WAVE == s1_lead_wave()) {   // the lead wave holds the tile's sorted 128 keys
        const int64_t o = ((int64_t)row * P.Zv + tile) * KMAX + (tid & (WAVE - 1));
        ((Key*)P.scratch)[o] = res.lo;
        ((Key*)P.scratch)[o + WAVE] = res.hi;
        if (P.out_ids) {
            auto id_of = [&](Key k) -> int {
                if (k == 0) return -1;
                const uint32_t lo = DT == SS_BF16 ? (0xFFFFu - ((uint32_t)k & 0xFFFFu))
                                                  : (0xFFFFFFFFu - (uint32_t)k);
                return tile * S1Traits<DT>::BN + (int)lo;
            };
            P.out_ids[o] = id_of(res.lo);
            P.out_ids[o + WAVE] = id_of(res.hi);
        }
    }
}

}  // namespace ssd
