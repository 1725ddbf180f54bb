// Speculative verification (SonicSampler section 3.1 "Speculative
// verification"; rejection-sampling rules of the decoding notes, "Rejection
// Sampler"): one workgroup per request walks its gamma draft positions in
// order.  Stage 2 has already reduced every target row to its kept
// candidates and truncated, renormalised probabilities p_j, so draft
// probabilities q_j are only gathered at the draft token and at the <= 128
// kept candidates; the residual max(0, p_j - q_j) vanishes outside them.
#pragma once

#include "ss_stage2.h"

namespace ssd {

constexpr int VF_THREADS = 128;

struct VerifyParams {
    int B;
    int gamma;
    int V;
    const RowRec* recs;
    const int32_t* draft_ids;
    const float* draft_probs;
    const ss_rng* rng;
    int32_t* out_tokens;
    int32_t* out_n_emit;
    int32_t* out_status;
};

__global__ __launch_bounds__(VF_THREADS) void verify_kernel(VerifyParams P) {
    __shared__ float s_redf[VF_THREADS / WAVE];
    __shared__ int s_redi[VF_THREADS / WAVE];
    __shared__ float s_pd;

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int G = P.gamma;
    const ss_rng rg = *P.rng;
    int32_t* out = P.out_tokens + (int64_t)b * (G + 1);
    for (int j = tid; j <= G; j += VF_THREADS) out[j] = -1;
    __syncthreads();

    const RowRec* r0 = P.recs + (int64_t)b * (G + 1);
    int emitted = 0;
    int st;
    if (r0->status == SS_ROW_INVALID) {
        st = SS_ROW_INVALID;
    } else {
        st = r0->status == SS_ROW_TOPK_CLAMPED ? SS_ROW_TOPK_CLAMPED : SS_ROW_OK;
        for (int j = 0; j <= G; ++j) {
            const RowRec* rec = r0 + j;
            if (rec->status == SS_ROW_ALL_MASKED) {
                st = SS_ROW_ALL_MASKED;
                break;
            }
            if (j == G) {   // every draft accepted: bonus token
                if (tid == 0) out[emitted] = rec->token;
                ++emitted;
                break;
            }
            const int d = P.draft_ids[(int64_t)b * G + j];
            if (rec->greedy) {
                const int a = rec->ids[0];
                if (tid == 0) out[emitted] = d == a ? d : a;
                ++emitted;
                if (d == a) continue;
                break;
            }
            const int n = rec->n;
            const float* q = P.draft_probs + ((int64_t)b * G + j) * P.V;
            if (tid == 0) s_pd = 0.0f;
            __syncthreads();
            if (tid < n && rec->ids[tid] == d) s_pd = rec->p[tid];
            __syncthreads();
            const float p_d = s_pd;
            const float q_d = (d >= 0 && d < P.V) ? q[d] : 0.0f;
            const float u = unit_open(philox_w0(rg.seed, rg.offset, 0u, (uint32_t)b, (1u << 24) | (uint32_t)j));
            if (q_d > 0.0f && u * q_d <= p_d) {
                if (tid == 0) out[emitted] = d;
                ++emitted;
                continue;
            }
            // rejected: draw from norm(max(0, p - q)) by Gumbel-max on ln(rho)
            const uint32_t c2 = (2u << 24) | (uint32_t)j;
            float s = 0.0f;
            bool ok = false;
            int id = -1;
            if (tid < n) {
                id = rec->ids[tid];
                const float rho = rec->p[tid] - q[id];
                if (rho > 0.0f) {
                    ok = true;
                    s = log_fixed(rho) + gumbel_noise(rg.seed, rg.offset, (uint32_t)id, (uint32_t)b, c2);
                }
            }
            int tok = block_argmax(s, id, ok, s_redf, s_redi);
            if (tok < 0) {   // p <= q on every kept candidate: draw from p
                const bool c = tid < n;
                float s2 = 0.0f;
                if (c) s2 = rec->v[tid] + gumbel_noise(rg.seed, rg.offset, (uint32_t)id, (uint32_t)b, c2);
                tok = block_argmax(s2, id, c, s_redf, s_redi);
            }
            if (tid == 0) out[emitted] = tok;
            ++emitted;
            break;
        }
    }
    if (tid == 0) {
        P.out_n_emit[b] = st == SS_ROW_INVALID ? 0 : emitted;
        if (P.out_status) P.out_status[b] = st;
    }
}

}  // namespace ssd
