// Speculative verification (SonicSampler section 3.1 "Speculative
// verification"; rejection-sampling rules of the decoding notes, "Rejection
// Sampler").  Stage 2 has already reduced every target row to its kept
// candidates and truncated, renormalised probabilities p_j, so draft
// probabilities q_j are only gathered at the draft token and at the <= 128
// kept candidates; the residual max(0, p_j - q_j) vanishes outside them.
//
// What happens at position j depends only on position j's data (accept or
// not, and the residual draw if not), so all positions are evaluated at
// once; one lane then walks them in order to emit the accepted prefix and
// the first rejection's draw (or the bonus token).  Up to 512 requests,
// Stage 2 does this itself (decide_position in each target row's
// workgroup; the request's last row to finish completes the output from
// the positions' bits); above that, verify_kernel does it with one
// workgroup per request from the rows' records (emit_request).
//
// With per-request draft counts (inclusive cumulative offsets, as the
// notes' rejection kernel reads its range from cu_num_draft_tokens),
// request b checks n_b = cu[b] - cu[b-1] drafts, at positions 0..n_b-1 of
// its gamma + 1 rows, and its bonus position is n_b; rows past n_b take no
// part.  A count outside [0, gamma] makes the request invalid.
#pragma once

#include "ss_stage2.h"

namespace ssd {

constexpr int VF_WAVES = 8;
constexpr int VF_THREADS = VF_WAVES * WAVE;

__global__ __launch_bounds__(VF_THREADS) void verify_kernel(Stage2Params F) {
    __shared__ int s_accept[SS_GAMMA_MAX + 1];
    __shared__ int s_token[SS_GAMMA_MAX + 1];
    __shared__ int s_status[SS_GAMMA_MAX + 1];
    const int b = blockIdx.x;
    const int lane = lane_id();
    const int wave = threadIdx.x / WAVE;
    const int G = F.gamma;
    const int V = F.s1.V;
    const ss_rng rg = *F.rng;
    const RowRec* r0 = F.recs + (int64_t)b * (G + 1);
    const DraftCount dc = draft_count(F, b);

    for (int j = wave; j <= dc.n; j += VF_WAVES) {
        const RowRec* rec = r0 + j;
        // every record field and draft value this position may use is
        // requested at once (no load waits on a branch), then the draft
        // probabilities at the candidates and at the draft token
        const int status = rec->status;
        const int greedy = rec->greedy;
        const int n = rec->n;
        const int rtoken = rec->token;
        const int best = rec->ids[0];
        const int d = j < dc.n ? F.draft_ids[(int64_t)b * G + j] : -1;
        const int id_lo_r = rec->ids[lane], id_hi_r = rec->ids[lane + 64];
        const float p_lo_r = rec->p[lane], p_hi_r = rec->p[lane + 64];
        const float v_lo = rec->v[lane], v_hi = rec->v[lane + 64];
        const float* q = F.draft_probs + ((int64_t)b * G + (j < G ? j : G - 1)) * V;   // any row for j = G
        auto in_v = [&](int id) { return (unsigned)id < (unsigned)V; };
        const float q_lo_r = q[in_v(id_lo_r) ? id_lo_r : 0];
        const float q_hi_r = q[in_v(id_hi_r) ? id_hi_r : 0];
        const float q_d_r = q[in_v(d) ? d : 0];
        const PosNoise nz = position_noise(rg, b, j, id_lo_r, id_hi_r);
        const PosDecision pd = decide_position(b, j, dc.n, status, greedy, n, rtoken, best, d, id_lo_r, id_hi_r,
                                               p_lo_r, p_hi_r, v_lo, v_hi, q_lo_r, q_hi_r, q_d_r, V, nz);
        if (lane == 0) {
            s_accept[j] = pd.accept;
            s_token[j] = pd.token;
            s_status[j] = status;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) emit_request(F, b, dc, s_accept, s_token, s_status);
}

}  // namespace ssd
