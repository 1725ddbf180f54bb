// Stage 2 (SonicSampler section 3.2 and Fig. 1, stage 2) for one row: the
// row's Z_v tile lists are re-indexed to global token ids and merged with
// bitonic merge networks into the row's 128 best tokens; then the fused
// epilogue runs: temperature, softmax weights, top-p / min-p truncation
// and Gumbel-max selection (section 3.1 "Probability truncation",
// "Sampling").
//
// Stage 2 runs inside the workgroup that finished the row's last tile (see
// ss_fused.h), so each row's merge overlaps other rows' Stage-1 streaming.
//
// Tokens named by an active penalty or bias list never enter the tiles;
// Stage 2 computes their processed logits directly (gather + the list
// arithmetic in list order) and merges them as one more sorted list.
//
// Merge key (64-bit, larger = better): ord32(z) << 32 | (0xFFFFFFFF - id).
#pragma once

#include "ss_stage1.h"

namespace ssd {

constexpr int S2_GROUP = 8;   // tile lists merged per LDS pass

enum { MODE_TILES = 0, MODE_SAMPLE = 1, MODE_VERIFY = 2, MODE_TOPK = 3 };

// Per target row, written in verification mode.
struct RowRec {
    int32_t ids[KMAX];   // candidates in order (-1 past K)
    float v[KMAX];       // z * (1/T), clamped
    float p[KMAX];       // e_k / E_n for kept ranks, else 0
    int32_t n;           // kept ranks
    int32_t K;
    int32_t token;       // greedy: best id; else Gumbel-max draw, counter {id, b, j}
    int32_t status;      // SS_ROW_*
    int32_t greedy;
    int32_t pad[3];
};

struct FusedParams {
    Stage1Params s1;
    const ss_rng* rng;
    int mode;
    int topk_k;
    uint32_t* row_cnt;   // [rows] tiles finished per row (kept at 0 between calls)
    uint32_t* req_cnt;   // [requests] rows finished per request (verification)
    // sampling outputs
    int32_t* tokens;
    int32_t* topk_ids;
    float* probs;
    int32_t* kept;
    float* mass;
    int32_t* status;
    // verification
    RowRec* recs;
    int gamma;
    const int32_t* draft_ids;
    const float* draft_probs;
    int32_t* v_tokens;
    int32_t* v_n_emit;
    int32_t* v_status;
    // top-k
    float* topk_vals;
};

struct S2Shared {
    uint64_t buf[S2_GROUP][KMAX];
    uint64_t acc[KMAX];
    uint64_t lkeys[S1_LIST_CAP];
    float redf[S1_WAVES];
    int redi[S1_WAVES];
    float pd;
};

struct RowParams {
    int valid;
    int greedy;
    int K;
    int clamped;
    uint32_t flags;
    float temperature;
    float top_p;
    float min_p;
    float rep;
    float freq;
    float pres;
    int n_prior;   // entries used (0 when the list does not apply)
    int n_bias;
};

__device__ __forceinline__ bool finitef(float x) { return x == x && x - x == 0.0f; }

// Row validation and parameters; every thread computes the same values from
// the (uniform) request record.
__device__ inline RowParams row_params(const Stage1Params& P, int b) {
    RowParams rp{};
    if (!P.req) {   // plain top-k: no processing
        rp.valid = 1;
        rp.greedy = 1;
        rp.K = min(KMAX, P.V);
        return rp;
    }
    const ss_req r = P.req[b];
    const uint32_t f = r.flags;
    rp.flags = f;
    rp.temperature = r.temperature;
    rp.top_p = r.top_p;
    rp.min_p = r.min_p;
    rp.rep = r.rep_penalty;
    rp.freq = r.freq_penalty;
    rp.pres = r.pres_penalty;
    bool ok = true;
    if ((int)r.n_prior > P.aux.prior_stride || (int)r.n_bias > P.aux.bias_stride) ok = false;
    if ((f & SS_GRAMMAR) && !P.aux.bitmask) ok = false;
    if ((f & (SS_REP | SS_FREQPRES)) && r.n_prior > 0 && (!P.aux.prior_ids || !P.aux.prior_cnt)) ok = false;
    if ((f & SS_BIAS) && r.n_bias > 0 && (!P.aux.bias_ids || !P.aux.bias_val)) ok = false;
    if ((f & SS_REP) && !(finitef(r.rep_penalty) && r.rep_penalty > 0.0f)) ok = false;
    if ((f & SS_FREQPRES) && !(finitef(r.freq_penalty) && finitef(r.pres_penalty))) ok = false;
    if (ok && (f & SS_BIAS)) {
        const float* bv = P.aux.bias_val + (int64_t)b * P.aux.bias_stride;
        bool fin = true;
        for (int j = 0; j < (int)r.n_bias; ++j) fin &= finitef(bv[j]);
        ok = fin;
    }
    bool g = (f & SS_GREEDY) != 0;
    if (!g) {
        if (r.temperature != r.temperature) ok = false;
        else if (r.temperature <= 0.0f) g = true;
        else if ((f & SS_TOPK) && r.top_k == 1) g = true;
    }
    if (!g) {
        if (!finitef(r.temperature)) ok = false;
        if ((f & SS_TOPK) && r.top_k < 1) ok = false;
        if ((f & SS_TOPP) && !(r.top_p > 0.0f && r.top_p <= 1.0f)) ok = false;
        if ((f & SS_MINP) && !(r.min_p >= 0.0f && r.min_p <= 1.0f)) ok = false;
    }
    rp.valid = ok;
    rp.greedy = g;
    int K = KMAX;
    if ((f & SS_TOPK) && r.top_k >= 1) {
        if (r.top_k > KMAX) rp.clamped = 1;
        else K = r.top_k;
    }
    rp.K = min(K, P.V);
    rp.n_prior = (f & (SS_REP | SS_FREQPRES)) ? (int)r.n_prior : 0;
    rp.n_bias = (f & SS_BIAS) ? (int)r.n_bias : 0;
    return rp;
}

template <int DT>
__device__ __forceinline__ uint64_t merge_key(typename S1Traits<DT>::Key e, int tile) {
    if (e == 0) return 0ull;
    uint32_t k32, local;
    if (DT == SS_BF16) {
        k32 = k16_to_k32((uint32_t)e >> 16);
        local = 0xFFFFu - ((uint32_t)e & 0xFFFFu);
    } else {
        k32 = (uint32_t)((uint64_t)e >> 32);
        local = 0xFFFFFFFFu - (uint32_t)e;
    }
    const uint32_t gid = (uint32_t)tile * (uint32_t)S1Traits<DT>::BN + local;
    return ((uint64_t)k32 << 32) | (uint64_t)(0xFFFFFFFFu - gid);
}

__device__ __forceinline__ int key_id(uint64_t k) { return k ? (int)(0xFFFFFFFFu - (uint32_t)k) : -1; }
__device__ __forceinline__ float key_z(uint64_t k) {
    return k ? unord32((uint32_t)(k >> 32)) : bitsf(F32_NINF_BITS);
}

// Merge sorted-descending lists A and B (128 each) into A: the elementwise
// max of A and reversed B is bitonic and holds the 128 best; seven
// half-cleaner steps sort it.  `npairs` merges run together; pair m uses
// lists slot(m) and slot(m) + stride.
__device__ __forceinline__ void merge_level(uint64_t (*buf)[KMAX], int npairs, int stride) {
    for (int idx = threadIdx.x; idx < npairs * KMAX; idx += S1_THREADS) {
        const int m = idx / KMAX, i = idx % KMAX;
        uint64_t* A = buf[m * 2 * stride];
        const uint64_t* Bl = buf[m * 2 * stride + stride];
        const uint64_t a = A[i], bb = Bl[KMAX - 1 - i];
        A[i] = a > bb ? a : bb;
    }
    __syncthreads();
    for (int j = KMAX / 2; j > 0; j >>= 1) {
        for (int idx = threadIdx.x; idx < npairs * (KMAX / 2); idx += S1_THREADS) {
            const int m = idx / (KMAX / 2), q = idx % (KMAX / 2);
            uint64_t* A = buf[m * 2 * stride];
            const int i = (q / j) * 2 * j + (q % j);
            const uint64_t a = A[i], c = A[i + j];
            if (a < c) {
                A[i] = c;
                A[i + j] = a;
            }
        }
        __syncthreads();
    }
}

// acc <- the 128 best of acc and B (both sorted descending).
__device__ __forceinline__ void merge_into(uint64_t* acc, const uint64_t* B) {
    if (threadIdx.x < KMAX) {
        const int i = threadIdx.x;
        const uint64_t a = acc[i], bb = B[KMAX - 1 - i];
        acc[i] = a > bb ? a : bb;
    }
    __syncthreads();
    for (int j = KMAX / 2; j > 0; j >>= 1) {
        if (threadIdx.x < KMAX / 2) {
            const int q = threadIdx.x;
            const int i = (q / j) * 2 * j + (q % j);
            const uint64_t a = acc[i], c = acc[i + j];
            if (a < c) {
                acc[i] = c;
                acc[i + j] = a;
            }
        }
        __syncthreads();
    }
}

// Wave-wide best (score desc, id asc); lanes with ok=false do not compete.
__device__ __forceinline__ int wave_argmax(float s, int id, bool ok) {
    float bs = s;
    int bi = ok ? id : -1;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float os = __shfl_xor(bs, o, WAVE);
        const int oi = __shfl_xor(bi, o, WAVE);
        const bool take = oi >= 0 && (bi < 0 || os > bs || (os == bs && oi < bi));
        if (take) {
            bs = os;
            bi = oi;
        }
    }
    return bi;
}

__device__ __forceinline__ float readlane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// The row's 128 best (merge keys, descending) into sh.acc.  Ends with a barrier.
template <int DT>
__device__ void row_merge(const FusedParams& F, const RowParams& rp, int row, int b, S2Shared& sh) {
    using Key = typename S1Traits<DT>::Key;
    const Stage1Params& P = F.s1;
    const int tid = threadIdx.x;

    // ---- listed tokens: exact processed logits, one sorted list ----
    const int np = rp.valid ? rp.n_prior : 0;
    const int nb = rp.valid ? rp.n_bias : 0;
    const int ncomb = np + nb;
    if (tid < KMAX) sh.acc[tid] = 0ull;
    if (ncomb > 0) {
        const int32_t* pid = P.aux.prior_ids + (int64_t)b * P.aux.prior_stride;
        const int32_t* pct = P.aux.prior_cnt + (int64_t)b * P.aux.prior_stride;
        const int32_t* bid = P.aux.bias_ids + (int64_t)b * P.aux.bias_stride;
        const float* bvl = P.aux.bias_val + (int64_t)b * P.aux.bias_stride;
        const bool grammar = (rp.flags & SS_GRAMMAR) != 0;
        for (int t0 = 0; t0 < ncomb; t0 += S1_THREADS) {   // uniform loop
            const int t = t0 + tid;
            int id = -1;
            bool ok = false;
            if (t < np) {
                id = pid[t];
                ok = pct[t] >= 1 && id >= 0 && id < P.V;
            } else if (t < ncomb) {
                id = bid[t - np];
                ok = id >= 0 && id < P.V;
            }
            float z = 0.0f;
            bool allowed = true;
            if (ok) {
                if (DT == SS_BF16) z = widen_bf16(((const uint16_t*)P.logits)[(int64_t)row * P.ld + id]);
                else z = ((const float*)P.logits)[(int64_t)row * P.ld + id];
                if (grammar)
                    allowed = (P.aux.bitmask[(int64_t)row * P.aux.bitmask_stride + (id >> 5)] >> (id & 31)) & 1u;
            }
            if (!allowed) z = bitsf(F32_NINF_BITS);
            // the list entries are the same for every lane: uniform loads
            bool dup = false;
            const bool do_rep = (rp.flags & SS_REP) != 0;
#pragma unroll 8
            for (int u = 0; u < np; ++u) {
                const bool m = pct[u] >= 1 && pid[u] == id;
                dup |= m && u < t;
                if (do_rep && m) z = (z > 0.0f) ? z / rp.rep : z * rp.rep;
            }
            if (rp.flags & SS_FREQPRES) {
#pragma unroll 8
                for (int u = 0; u < np; ++u) {
                    const int c = pct[u];
                    if (c >= 1 && pid[u] == id) {
                        const float pen = (float)c * rp.freq + rp.pres;
                        z = z - pen;
                    }
                }
            }
#pragma unroll 8
            for (int u = 0; u < nb; ++u) {
                const bool m = bid[u] == id;
                dup |= m && np + u < t;
                if (m) z = z + bvl[u];
            }
            if (t < ncomb)
                sh.lkeys[t] = (ok && !dup)
                                  ? (((uint64_t)ord32(canon(z)) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id))
                                  : 0ull;
        }
        int Pl = KMAX;
        while (Pl < ncomb) Pl <<= 1;
        for (int t = ncomb + tid; t < Pl; t += S1_THREADS) sh.lkeys[t] = 0ull;
        __syncthreads();
        block_sort_desc<uint64_t, S1_THREADS>(sh.lkeys, Pl);
        if (tid < KMAX) sh.acc[tid] = sh.lkeys[tid];
    }
    __syncthreads();

    // ---- tile lists: load a group, merge it down to one list, fold into acc ----
    const Key* sc = (const Key*)P.scratch + (int64_t)row * P.Zv * KMAX;
    for (int g0 = 0; g0 < P.Zv; g0 += S2_GROUP) {
        const int G = min(S2_GROUP, P.Zv - g0);
        for (int idx = tid; idx < G * KMAX; idx += S1_THREADS) {
            const int l = idx / KMAX, i = idx % KMAX;
            sh.buf[l][i] = merge_key<DT>(sc[(int64_t)(g0 + l) * KMAX + i], g0 + l);
        }
        __syncthreads();
        for (int s = 1; s < G; s <<= 1) {
            const int npairs = (G - s + 2 * s - 1) / (2 * s);   // m with m*2s + s < G
            merge_level(sh.buf, npairs, s);
        }
        merge_into(sh.acc, sh.buf[0]);
    }
}

// Epilogue on wave 0 (ranks k = lane and lane + 64).  Writes the mode's
// outputs for the row.  Uses no barrier.
template <int DT>
__device__ void row_epilogue(const FusedParams& F, const RowParams& rp, int row, int b, S2Shared& sh) {
    const Stage1Params& P = F.s1;
    const int lane = lane_id();
    const uint64_t k_lo = sh.acc[lane], k_hi = sh.acc[lane + 64];
    const int id_lo = key_id(k_lo), id_hi = key_id(k_hi);
    const float z_lo = key_z(k_lo), z_hi = key_z(k_hi);
    const uint64_t k0 = sh.acc[0];
    const int id0 = key_id(k0);
    const float z0 = key_z(k0);
    const float NINF = bitsf(F32_NINF_BITS);

    if (F.mode == MODE_TOPK) {
        const int kk = F.topk_k;
        for (int h = 0; h < 2; ++h) {
            const int k = lane + 64 * h;
            const int id = h ? id_hi : id_lo;
            if (k < kk) {
                const bool have = k < P.V && id >= 0;
                F.topk_ids[(int64_t)row * kk + k] = have ? id : -1;
                if (F.topk_vals) F.topk_vals[(int64_t)row * kk + k] = have ? (h ? z_hi : z_lo) : NINF;
            }
        }
        return;
    }

    const int K = rp.K;
    int status = SS_ROW_OK;
    if (!rp.valid) status = SS_ROW_INVALID;
    else if (z0 == NINF) status = SS_ROW_ALL_MASKED;
    else if (rp.clamped) status = SS_ROW_TOPK_CLAMPED;
    const bool live = status == SS_ROW_OK || status == SS_ROW_TOPK_CLAMPED;

    int token = -1, n = 0;
    float v_lo = NINF, v_hi = NINF, e_lo = 0.0f, e_hi = 0.0f, Z = 1.0f, En = 0.0f;
    if (live && rp.greedy) {
        token = id0;
        n = 1;
    } else if (live) {
        const float invT = 1.0f / rp.temperature;
        const float FMAX = bitsf(F32_MAX_BITS);
        auto vscale = [&](float z) -> float {
            if (z == NINF) return z;
            float v = z * invT;
            v = v > FMAX ? FMAX : v;
            v = v < -FMAX ? -FMAX : v;
            return v;
        };
        const float m = vscale(z0);
        if (lane < K) {
            v_lo = vscale(z_lo);
            e_lo = exp_fixed(v_lo - m);
        }
        if (lane + 64 < K) {
            v_hi = vscale(z_hi);
            e_hi = exp_fixed(v_hi - m);
        }
        // running sums E_k = e_0 + ... + e_{k-1}, left to right
        float E = 0.0f, E_lo = 0.0f, E_hi = 0.0f;
        const int k1 = min(K, 64);
        for (int k = 0; k < k1; ++k) {
            if (lane == k) E_lo = E;
            E = E + readlane_f(e_lo, k);
        }
        for (int k = 64; k < K; ++k) {
            if (lane == k - 64) E_hi = E;
            E = E + readlane_f(e_hi, k - 64);
        }
        Z = E;
        int n_p = K, n_m = K;
        if ((rp.flags & SS_TOPP) && rp.top_p < 1.0f) {
            const float thr = rp.top_p * Z;
            n_p = __popcll(__ballot(lane < K && E_lo < thr)) + __popcll(__ballot(lane + 64 < K && E_hi < thr));
        }
        if ((rp.flags & SS_MINP) && rp.min_p > 0.0f) {
            const float L = log_fixed(rp.min_p);
            n_m = __popcll(__ballot(lane < K && (v_lo - m) >= L)) +
                  __popcll(__ballot(lane + 64 < K && (v_hi - m) >= L));
        }
        n = min(n_p, n_m);
        // E_n: the running sum before rank n (Z when n = K)
        if (n >= K) En = Z;
        else if (n < 64) En = readlane_f(E_lo, n);
        else En = readlane_f(E_hi, n - 64);
        uint32_t c1, c2;
        if (F.mode == MODE_VERIFY) {
            c1 = (uint32_t)b;
            c2 = (uint32_t)(row - b * P.rows_per_req);
        } else {
            c1 = (uint32_t)row;
            c2 = 0u;
        }
        const ss_rng rg = *F.rng;
        float s_lo = 0.0f, s_hi = 0.0f;
        const bool c_lo = lane < n, c_hi = lane + 64 < n;
        if (c_lo) s_lo = v_lo + gumbel_noise(rg.seed, rg.offset, (uint32_t)id_lo, c1, c2);
        if (c_hi) s_hi = v_hi + gumbel_noise(rg.seed, rg.offset, (uint32_t)id_hi, c1, c2);
        // best of the lane's two, then across the wave
        float s = s_lo;
        int id = c_lo ? id_lo : -1;
        if (c_hi && (id < 0 || s_hi > s || (s_hi == s && id_hi < id))) {
            s = s_hi;
            id = id_hi;
        }
        token = wave_argmax(s, id, id >= 0);
    }

    if (F.mode == MODE_SAMPLE) {
        if (lane == 0) {
            F.tokens[row] = token;
            if (F.status) F.status[row] = status;
            if (F.kept) F.kept[row] = live ? n : 0;
            if (F.mass) F.mass[row] = live ? (rp.greedy ? 1.0f : En / Z) : 0.0f;
        }
        for (int h = 0; h < 2; ++h) {
            const int k = lane + 64 * h;
            if (F.topk_ids)
                F.topk_ids[(int64_t)row * KMAX + k] = (status != SS_ROW_INVALID && k < K) ? (h ? id_hi : id_lo) : -1;
            if (F.probs) {
                float pk = 0.0f;
                if (live) pk = rp.greedy ? (k == 0 ? 1.0f : 0.0f) : (k < K ? (h ? e_hi : e_lo) / Z : 0.0f);
                F.probs[(int64_t)row * KMAX + k] = pk;
            }
        }
    } else {   // MODE_VERIFY
        RowRec* rec = F.recs + row;
        for (int h = 0; h < 2; ++h) {
            const int k = lane + 64 * h;
            rec->ids[k] = (status != SS_ROW_INVALID && k < K) ? (h ? id_hi : id_lo) : -1;
            rec->v[k] = h ? v_hi : v_lo;
            rec->p[k] = (live && !rp.greedy && k < n) ? (h ? e_hi : e_lo) / En : 0.0f;
        }
        if (lane == 0) {
            rec->n = live ? n : 0;
            rec->K = K;
            rec->token = token;
            rec->status = status;
            rec->greedy = rp.greedy;
        }
    }
}

}  // namespace ssd
