// Speculative verification (SonicSampler section 3.1 "Speculative
// verification"; rejection-sampling rules of the decoding notes, "Rejection
// Sampler") for one request, on one wave.  Stage 2 has already reduced
// every target row to its kept candidates and truncated, renormalised
// probabilities p_j, so draft probabilities q_j are only gathered at the
// draft token and at the <= 128 kept candidates; the residual
// max(0, p_j - q_j) vanishes outside them.
#pragma once

#include "ss_stage2.h"

namespace ssd {

// Runs on wave 0 of the workgroup; lanes hold candidate ranks lane and
// lane + 64.  Uses no barrier.
__device__ void verify_request(const FusedParams& F, int b) {
    const int lane = lane_id();
    const int G = F.gamma;
    const int V = F.s1.V;
    const ss_rng rg = *F.rng;
    int32_t* out = F.v_tokens + (int64_t)b * (G + 1);
    if (lane == 0)
        for (int j = 0; j <= G; ++j) out[j] = -1;

    const RowRec* r0 = F.recs + (int64_t)b * (G + 1);
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
                if (lane == 0) out[emitted] = rec->token;
                ++emitted;
                break;
            }
            const int d = F.draft_ids[(int64_t)b * G + j];
            if (rec->greedy) {
                const int a = rec->ids[0];
                if (lane == 0) out[emitted] = d == a ? d : a;
                ++emitted;
                if (d == a) continue;
                break;
            }
            const int n = rec->n;
            const float* q = F.draft_probs + ((int64_t)b * G + j) * V;
            const int id_lo = lane < n ? rec->ids[lane] : -1;
            const int id_hi = lane + 64 < n ? rec->ids[lane + 64] : -1;
            const float p_lo = lane < n ? rec->p[lane] : 0.0f;
            const float p_hi = lane + 64 < n ? rec->p[lane + 64] : 0.0f;
            // p_j(d): the kept candidate equal to d, if any (ids are unique)
            float pd = 0.0f;
            const uint64_t m_lo = __ballot(id_lo == d && id_lo >= 0);
            const uint64_t m_hi = __ballot(id_hi == d && id_hi >= 0);
            if (m_lo) pd = readlane_f(p_lo, __builtin_ctzll(m_lo));
            else if (m_hi) pd = readlane_f(p_hi, __builtin_ctzll(m_hi));
            const float qd = (d >= 0 && d < V) ? q[d] : 0.0f;
            const float u = unit_open(philox_w0(rg.seed, rg.offset, 0u, (uint32_t)b, (1u << 24) | (uint32_t)j));
            if (qd > 0.0f && u * qd <= pd) {
                if (lane == 0) out[emitted] = d;
                ++emitted;
                continue;
            }
            // rejected: draw from norm(max(0, p - q)) by Gumbel-max on ln(rho)
            const uint32_t c2 = (2u << 24) | (uint32_t)j;
            float s_lo = 0.0f, s_hi = 0.0f;
            bool ok_lo = false, ok_hi = false;
            if (id_lo >= 0) {
                const float rho = p_lo - q[id_lo];
                if (rho > 0.0f) {
                    ok_lo = true;
                    s_lo = log_fixed(rho) + gumbel_noise(rg.seed, rg.offset, (uint32_t)id_lo, (uint32_t)b, c2);
                }
            }
            if (id_hi >= 0) {
                const float rho = p_hi - q[id_hi];
                if (rho > 0.0f) {
                    ok_hi = true;
                    s_hi = log_fixed(rho) + gumbel_noise(rg.seed, rg.offset, (uint32_t)id_hi, (uint32_t)b, c2);
                }
            }
            float s = s_lo;
            int id = ok_lo ? id_lo : -1;
            if (ok_hi && (id < 0 || s_hi > s || (s_hi == s && id_hi < id))) {
                s = s_hi;
                id = id_hi;
            }
            int tok = wave_argmax(s, id, id >= 0);
            if (tok < 0) {   // p <= q on every kept candidate: draw from p
                s_lo = 0.0f;
                s_hi = 0.0f;
                if (id_lo >= 0) s_lo = rec->v[lane] + gumbel_noise(rg.seed, rg.offset, (uint32_t)id_lo, (uint32_t)b, c2);
                if (id_hi >= 0)
                    s_hi = rec->v[lane + 64] + gumbel_noise(rg.seed, rg.offset, (uint32_t)id_hi, (uint32_t)b, c2);
                s = s_lo;
                id = id_lo;
                if (id_hi >= 0 && (id < 0 || s_hi > s || (s_hi == s && id_hi < id))) {
                    s = s_hi;
                    id = id_hi;
                }
                tok = wave_argmax(s, id, id >= 0);
            }
            if (lane == 0) out[emitted] = tok;
            ++emitted;
            break;
        }
    }
    if (st == SS_ROW_INVALID) emitted = 0;
    if (lane == 0) {
        F.v_n_emit[b] = emitted;
        if (F.v_status) F.v_status[b] = st;
    }
}

}  // namespace ssd
