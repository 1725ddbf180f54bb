// One launch for the whole step.  Every workgroup runs Stage 1 on its
// (row, tile) and writes the tile's 128 keys to the workspace; the
// workgroup that finishes a row's last tile (per-row counter, release /
// acquire at device scope) runs Stage 2 for that row, so each row's merge
// and epilogue overlap the streaming of the other rows.  In verification
// mode the last row of a request to finish runs that request's draft
// verification the same way.  Counters are returned to zero by the last
// arriver, so the workspace stays ready for the next call (and for graph
// replays) without any memset.
#pragma once

#include "ss_verify.h"

namespace ssd {

template <int DT>
union FusedShared {
    S1Shared<DT> s1;
    S2Shared s2;
};

// Increment *cnt; true for the caller that brings it to `total` (which
// also resets it to 0).  The counter update is performed at system scope so
// it is coherent across the XCDs' separate L2 caches; the callers fence
// (write back / invalidate L2) around it at device scope.
__device__ __forceinline__ bool arrive_last(uint32_t* cnt, uint32_t total) {
    const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_SYSTEM);
    const bool last = old == total - 1u;
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    return last;
}

template <int DT, int MODE>
__global__ __launch_bounds__(S1_THREADS) void fused_kernel(FusedParams F) {
    using Key = typename S1Traits<DT>::Key;
    __shared__ FusedShared<DT> sh;
    __shared__ int s_last;
    const Stage1Params& P = F.s1;
    const int tid = threadIdx.x;
    const int row = blockIdx.x / P.Zv;
    const int tile = blockIdx.x - row * P.Zv;

    stage1_tile<DT>(P, row, tile, sh.s1);
    if (tid < KMAX) {
        const int64_t o = ((int64_t)row * P.Zv + tile) * KMAX + tid;
        const Key k = sh.s1.surv[tid];
        ((Key*)P.scratch)[o] = k;
        if (MODE == MODE_TILES && P.out_ids) {
            int id = -1;
            if (k != 0) {
                const uint32_t lo = DT == SS_BF16 ? (0xFFFFu - ((uint32_t)k & 0xFFFFu))
                                                  : (0xFFFFFFFFu - (uint32_t)k);
                id = tile * S1Traits<DT>::BN + (int)lo;
            }
            P.out_ids[o] = id;
        }
    }
    if (MODE == MODE_TILES) return;

    // ---- the last tile of the row to finish runs Stage 2 ----
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = arrive_last(F.row_cnt + row, (uint32_t)P.Zv);
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    const int b = row / P.rows_per_req;
    const RowParams rp = row_params(P, b);
    row_merge<DT>(F, rp, row, b, sh.s2);
    if (tid >= WAVE) return;   // the epilogue and verification run on wave 0
    row_epilogue<DT>(F, rp, row, b, sh.s2);
    if (MODE != MODE_VERIFY) return;

    // ---- the last row of the request to finish verifies its drafts ----
    __threadfence();
    int lastreq = 0;
    if (tid == 0) lastreq = arrive_last(F.req_cnt + b, (uint32_t)P.rows_per_req);
    lastreq = __shfl(lastreq, 0, WAVE);
    if (!lastreq) return;
    __threadfence();
    verify_request(F, b);
}

}  // namespace ssd
