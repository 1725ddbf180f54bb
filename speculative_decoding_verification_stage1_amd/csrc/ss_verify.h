// Speculative verification (SonicSampler section 3.1 "Speculative
// verification"; rejection-sampling rules of the decoding notes, "Rejection
// Sampler").  Stage 2 has already reduced every target row to its kept
// candidates and truncated, renormalised probabilities p_j, so draft
// probabilities q_j are only gathered at the draft token and at the <= 128
// kept candidates; the residual max(0, p_j - q_j) vanishes outside them.
//
// One workgroup per request.  What happens at position j depends only on
// position j's data (accept or not, and the residual draw if not), so the
// waves evaluate all positions at once; one lane then walks the positions
// in order to emit the accepted prefix and the first rejection's draw (or
// the bonus token).
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
    int Gb = G;   // this request's draft count (uniform)
    bool count_ok = true;
    if (F.cu_num_draft) {
        const int hi = F.cu_num_draft[b];
        const int lo = b > 0 ? F.cu_num_draft[b - 1] : 0;
        count_ok = hi - lo >= 0 && hi - lo <= G;
        Gb = count_ok ? hi - lo : 0;
    }

    for (int j = wave; j <= Gb; j += VF_WAVES) {
        const RowRec* rec = r0 + j;
        // every record field and draft value this position may use is
        // requested at once (no load waits on a branch), then the draft
        // probabilities at the candidates and at the draft token
        const int status = rec->status;
        const int greedy = rec->greedy;
        const int n = rec->n;
        const int rtoken = rec->token;
        const int best = rec->ids[0];
        const int d = j < Gb ? F.draft_ids[(int64_t)b * G + j] : -1;
        const int id_lo_r = rec->ids[lane], id_hi_r = rec->ids[lane + 64];
        const float p_lo_r = rec->p[lane], p_hi_r = rec->p[lane + 64];
        const float v_lo = rec->v[lane], v_hi = rec->v[lane + 64];
        const float* q = F.draft_probs + ((int64_t)b * G + (j < G ? j : G - 1)) * V;   // any row for j = G
        auto in_v = [&](int id) { return (unsigned)id < (unsigned)V; };
        const float q_lo_r = q[in_v(id_lo_r) ? id_lo_r : 0];
        const float q_hi_r = q[in_v(id_hi_r) ? id_hi_r : 0];
        const float q_d_r = q[in_v(d) ? d : 0];
        int accept = 0, token = -1;
        const bool live = status == SS_ROW_OK || status == SS_ROW_TOPK_CLAMPED;
        if (live && j == Gb) {         // bonus token
            token = rtoken;
            accept = 1;
        } else if (live && greedy) {
            token = best;
            accept = d == token;
        } else if (live) {
            const int id_lo = lane < n ? id_lo_r : -1;
            const int id_hi = lane + 64 < n ? id_hi_r : -1;
            const float p_lo = lane < n ? p_lo_r : 0.0f;
            const float p_hi = lane + 64 < n ? p_hi_r : 0.0f;
            const float q_lo = id_lo >= 0 ? q_lo_r : 0.0f;
            const float q_hi = id_hi >= 0 ? q_hi_r : 0.0f;
            const float qd = (d >= 0 && d < V) ? q_d_r : 0.0f;
            // p_j(d): the kept candidate equal to d, if any (ids are unique)
            float pd = 0.0f;
            const uint64_t m_lo = __ballot(id_lo == d && id_lo >= 0);
            const uint64_t m_hi = __ballot(id_hi == d && id_hi >= 0);
            if (m_lo) pd = readlane_f(p_lo, __builtin_ctzll(m_lo));
            else if (m_hi) pd = readlane_f(p_hi, __builtin_ctzll(m_hi));
            const float u = unit_open(philox_w0(rg.seed, rg.offset, 0u, (uint32_t)b, (1u << 24) | (uint32_t)j));
            accept = qd > 0.0f && u * qd <= pd;
            if (!accept) {
                // draw from norm(max(0, p - q)) by Gumbel-max on ln(rho)
                const uint32_t c2 = (2u << 24) | (uint32_t)j;
                const float g_lo =
                    id_lo >= 0 ? gumbel_noise(rg.seed, rg.offset, (uint32_t)id_lo, (uint32_t)b, c2) : 0.0f;
                const float g_hi =
                    id_hi >= 0 ? gumbel_noise(rg.seed, rg.offset, (uint32_t)id_hi, (uint32_t)b, c2) : 0.0f;
                const float rho_lo = p_lo - q_lo, rho_hi = p_hi - q_hi;
                const bool ok_lo = id_lo >= 0 && rho_lo > 0.0f;
                const bool ok_hi = id_hi >= 0 && rho_hi > 0.0f;
                float s = ok_lo ? log_fixed(rho_lo) + g_lo : 0.0f;
                int id = ok_lo ? id_lo : -1;
                if (ok_hi) {
                    const float sh = log_fixed(rho_hi) + g_hi;
                    if (id < 0 || sh > s || (sh == s && id_hi < id)) {
                        s = sh;
                        id = id_hi;
                    }
                }
                token = wave_argmax(s, id, id >= 0);
                if (token < 0) {   // p <= q on every kept candidate: draw from p
                    float s2 = id_lo >= 0 ? v_lo + g_lo : 0.0f;
                    int i2 = id_lo;
                    if (id_hi >= 0) {
                        const float sh = v_hi + g_hi;
                        if (i2 < 0 || sh > s2 || (sh == s2 && id_hi < i2)) {
                            s2 = sh;
                            i2 = id_hi;
                        }
                    }
                    token = wave_argmax(s2, i2, i2 >= 0);
                }
            }
        }
        if (lane == 0) {
            s_accept[j] = accept;
            s_token[j] = token;
            s_status[j] = status;
        }
    }
    __syncthreads();

    if (threadIdx.x == 0) {
        int32_t* out = F.v_tokens + (int64_t)b * (G + 1);
        int emitted = 0;
        int st;
        if (!count_ok || s_status[0] == SS_ROW_INVALID) {
            st = SS_ROW_INVALID;
        } else {
            st = s_status[0] == SS_ROW_TOPK_CLAMPED ? SS_ROW_TOPK_CLAMPED : SS_ROW_OK;
            for (int j = 0; j <= Gb; ++j) {
                if (s_status[j] == SS_ROW_ALL_MASKED) {
                    st = SS_ROW_ALL_MASKED;
                    break;
                }
                if (j < Gb && s_accept[j]) {
                    out[emitted++] = F.draft_ids[(int64_t)b * G + j];
                    continue;
                }
                out[emitted++] = s_token[j];   // first rejection's draw, or the bonus
                break;
            }
        }
        for (int j = emitted; j <= G; ++j) out[j] = -1;
        F.v_n_emit[b] = emitted;
        if (F.v_status) F.v_status[b] = st;
    }
}

}  // namespace ssd
