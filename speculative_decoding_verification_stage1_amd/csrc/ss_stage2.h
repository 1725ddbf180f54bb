// Stage 2 (SonicSampler section 3.2 and Fig. 1, stage 2): one workgroup per
// row gathers the row's Z_v tile lists, re-indexes them to global token ids,
// merges them with bitonic merge networks into the row's 128 best tokens,
// and runs the fused epilogue: temperature, softmax weights, top-p / min-p
// truncation and Gumbel-max selection (section 3.1 "Probability
// truncation", "Sampling").
//
// Tokens named by an active penalty or bias list never enter the tiles;
// Stage 2 computes their processed logits directly (gather + the list
// arithmetic in list order) and merges them as one more sorted list.
//
// Merge key (64-bit, larger = better): ord32(z) << 32 | (0xFFFFFFFF - id).
#pragma once

#include "ss_stage1.h"

namespace ssd {

constexpr int S2_THREADS = 256;
constexpr int S2_WAVES = S2_THREADS / WAVE;
constexpr int S2_GROUP = 32;   // tile lists merged per LDS pass

enum { MODE_SAMPLE = 0, MODE_VERIFY = 1, MODE_TOPK = 2 };

// Per target row, written by Stage 2 in verification mode.
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

struct Stage2Params {
    const void* logits;
    int64_t ld;
    int V;
    int rows;
    int Zv;
    int rows_per_req;
    const ss_req* req;
    ss_aux aux;
    const ss_rng* rng;
    const void* scratch;
    int mode;
    int topk_k;
    int32_t* tokens;
    int32_t* topk_ids;
    float* probs;
    int32_t* kept;
    float* mass;
    int32_t* status;
    RowRec* recs;
    float* topk_vals;
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

// Row validation and parameters (one thread).
__device__ inline RowParams row_params(const Stage2Params& P, int b) {
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
        for (int j = 0; j < (int)r.n_bias; ++j)
            if (!finitef(bv[j])) ok = false;
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

// Merge sorted-descending lists A and B (128 each) into A: the elementwise
// max of A and reversed B is bitonic and holds the 128 best; seven
// half-cleaner steps sort it.  `npairs` merges run together; pair m uses
// lists slot(m) and slot(m) + stride.
__device__ __forceinline__ void merge_level(uint64_t (*buf)[KMAX], int npairs, int stride) {
    for (int idx = threadIdx.x; idx < npairs * KMAX; idx += S2_THREADS) {
        const int m = idx / KMAX, i = idx % KMAX;
        uint64_t* A = buf[m * 2 * stride];
        const uint64_t* Bl = buf[m * 2 * stride + stride];
        const uint64_t a = A[i], bb = Bl[KMAX - 1 - i];
        A[i] = a > bb ? a : bb;
    }
    __syncthreads();
    for (int j = KMAX / 2; j > 0; j >>= 1) {
        for (int idx = threadIdx.x; idx < npairs * (KMAX / 2); idx += S2_THREADS) {
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

// Best (score desc, id asc) across the block; invalid lanes pass ok=false.
__device__ __forceinline__ int block_argmax(float s, int id, bool ok, float* ws, int* wi) {
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
    const int w = threadIdx.x / WAVE;
    if (lane_id() == 0) {
        ws[w] = bs;
        wi[w] = bi;
    }
    __syncthreads();
    float rs = ws[0];
    int ri = wi[0];
    for (int i = 1; i < (int)(blockDim.x / WAVE); ++i) {
        const float os = ws[i];
        const int oi = wi[i];
        if (oi >= 0 && (ri < 0 || os > rs || (os == rs && oi < ri))) {
            rs = os;
            ri = oi;
        }
    }
    __syncthreads();
    return ri;
}

__device__ __forceinline__ int block_count(bool c, int* tmp) {
    const uint64_t bal = __ballot(c);
    const int w = threadIdx.x / WAVE;
    if (lane_id() == 0) tmp[w] = __popcll(bal);
    __syncthreads();
    int t = 0;
    for (int i = 0; i < (int)(blockDim.x / WAVE); ++i) t += tmp[i];
    __syncthreads();
    return t;
}

template <int DT>
__global__ __launch_bounds__(S2_THREADS) void stage2_kernel(Stage2Params P) {
    using Key = typename S1Traits<DT>::Key;
    __shared__ uint64_t buf[S2_GROUP][KMAX];
    __shared__ uint64_t acc[KMAX];
    __shared__ uint64_t lkeys[S1_LIST_CAP];
    __shared__ int32_t s_pid[256], s_pcnt[256], s_bid[256];
    __shared__ float s_bval[256];
    __shared__ float s_e[KMAX];
    __shared__ float s_E[KMAX + 1];
    __shared__ float s_redf[S2_WAVES];
    __shared__ int s_redi[S2_WAVES];
    __shared__ RowParams s_rp;

    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    const int b = row / P.rows_per_req;
    if (tid == 0) s_rp = row_params(P, b);
    __syncthreads();
    const RowParams rp = s_rp;

    // ---- listed tokens: exact processed logits, as one sorted list ----
    const int np = rp.valid ? rp.n_prior : 0;
    const int nb = rp.valid ? rp.n_bias : 0;
    for (int j = tid; j < np; j += S2_THREADS) {
        s_pid[j] = P.aux.prior_ids[(int64_t)b * P.aux.prior_stride + j];
        s_pcnt[j] = P.aux.prior_cnt[(int64_t)b * P.aux.prior_stride + j];
    }
    for (int j = tid; j < nb; j += S2_THREADS) {
        s_bid[j] = P.aux.bias_ids[(int64_t)b * P.aux.bias_stride + j];
        s_bval[j] = P.aux.bias_val[(int64_t)b * P.aux.bias_stride + j];
    }
    for (int i = tid; i < KMAX; i += S2_THREADS) acc[i] = 0ull;
    __syncthreads();
    const int ncomb = np + nb;
    if (ncomb > 0) {
        const bool grammar = (rp.flags & SS_GRAMMAR) != 0;
        for (int t = tid; t < ncomb; t += S2_THREADS) {
            int id;
            bool ok;
            if (t < np) {
                id = s_pid[t];
                ok = s_pcnt[t] >= 1 && id >= 0 && id < P.V;
            } else {
                id = s_bid[t - np];
                ok = id >= 0 && id < P.V;
            }
            for (int u = 0; u < t && ok; ++u) {   // keep the first entry of each id
                const bool uok = u < np ? (s_pcnt[u] >= 1 && s_pid[u] == id) : (s_bid[u - np] == id);
                if (uok) ok = false;
            }
            uint64_t key = 0ull;
            if (ok) {
                float z;
                if (DT == SS_BF16) z = widen_bf16(((const uint16_t*)P.logits)[(int64_t)row * P.ld + id]);
                else z = ((const float*)P.logits)[(int64_t)row * P.ld + id];
                if (grammar && !((P.aux.bitmask[(int64_t)row * P.aux.bitmask_stride + (id >> 5)] >> (id & 31)) & 1u))
                    z = bitsf(F32_NINF_BITS);
                if (rp.flags & SS_REP)
                    for (int j = 0; j < np; ++j)
                        if (s_pcnt[j] >= 1 && s_pid[j] == id) z = (z > 0.0f) ? z / rp.rep : z * rp.rep;
                if (rp.flags & SS_FREQPRES)
                    for (int j = 0; j < np; ++j)
                        if (s_pcnt[j] >= 1 && s_pid[j] == id) {
                            const float pen = (float)s_pcnt[j] * rp.freq + rp.pres;
                            z = z - pen;
                        }
                if (rp.flags & SS_BIAS)
                    for (int j = 0; j < nb; ++j)
                        if (s_bid[j] == id) z = z + s_bval[j];
                key = ((uint64_t)ord32(canon(z)) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
            }
            lkeys[t] = key;
        }
        int Pl = KMAX;
        while (Pl < ncomb) Pl <<= 1;
        for (int t = ncomb + tid; t < Pl; t += S2_THREADS) lkeys[t] = 0ull;
        __syncthreads();
        block_sort_desc<uint64_t, S2_THREADS>(lkeys, Pl);
        for (int i = tid; i < KMAX; i += S2_THREADS) acc[i] = lkeys[i];
        __syncthreads();
    }

    // ---- tile lists: load a group, merge it down to one list, fold into acc ----
    const Key* sc = (const Key*)P.scratch + (int64_t)row * P.Zv * KMAX;
    for (int g0 = 0; g0 < P.Zv; g0 += S2_GROUP) {
        const int G = min(S2_GROUP, P.Zv - g0);
        for (int idx = tid; idx < G * KMAX; idx += S2_THREADS) {
            const int l = idx / KMAX, i = idx % KMAX;
            buf[l][i] = merge_key<DT>(sc[(int64_t)(g0 + l) * KMAX + i], g0 + l);
        }
        __syncthreads();
        for (int s = 1; s < G; s <<= 1) {
            const int npairs = (G - s + 2 * s - 1) / (2 * s);   // m with m*2s + s < G
            merge_level(buf, npairs, s);
        }
        // acc <- merge(acc, buf[0])
        for (int i = tid; i < KMAX; i += S2_THREADS) {
            const uint64_t a = acc[i], bb = buf[0][KMAX - 1 - i];
            acc[i] = a > bb ? a : bb;
        }
        __syncthreads();
        for (int j = KMAX / 2; j > 0; j >>= 1) {
            for (int q = tid; q < KMAX / 2; q += S2_THREADS) {
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

    // ---- epilogue: threads 0..127 hold rank k = tid ----
    const int k = tid;
    const bool lane_k = k < KMAX;
    uint64_t key = lane_k ? acc[k] : 0ull;
    const int id_k = key ? (int)(0xFFFFFFFFu - (uint32_t)key) : -1;
    const float z_k = key ? unord32((uint32_t)(key >> 32)) : bitsf(F32_NINF_BITS);
    const uint64_t key0 = acc[0];
    const int id0 = key0 ? (int)(0xFFFFFFFFu - (uint32_t)key0) : -1;
    const float z0 = key0 ? unord32((uint32_t)(key0 >> 32)) : bitsf(F32_NINF_BITS);

    if (P.mode == MODE_TOPK) {
        const int kk = P.topk_k;
        if (k < kk) {
            const bool have = k < P.V && id_k >= 0;
            P.topk_ids[(int64_t)row * kk + k] = have ? id_k : -1;
            if (P.topk_vals) P.topk_vals[(int64_t)row * kk + k] = have ? z_k : bitsf(F32_NINF_BITS);
        }
        return;
    }

    const int K = rp.K;
    int status = SS_ROW_OK;
    if (!rp.valid) status = SS_ROW_INVALID;
    else if (z0 == bitsf(F32_NINF_BITS)) status = SS_ROW_ALL_MASKED;
    else if (rp.clamped) status = SS_ROW_TOPK_CLAMPED;
    const bool live = status == SS_ROW_OK || status == SS_ROW_TOPK_CLAMPED;

    int token = -1, n = 0;
    float vk = bitsf(F32_NINF_BITS), ek = 0.0f, Z = 1.0f, En = 0.0f;
    if (live && rp.greedy) {
        token = id0;
        n = 1;
    } else if (live) {
        const float invT = 1.0f / rp.temperature;
        auto vscale = [&](float z) -> float {
            if (z == bitsf(F32_NINF_BITS)) return z;
            float v = z * invT;
            v = v > bitsf(F32_MAX_BITS) ? bitsf(F32_MAX_BITS) : v;
            v = v < -bitsf(F32_MAX_BITS) ? -bitsf(F32_MAX_BITS) : v;
            return v;
        };
        const float m = vscale(z0);
        if (k < K) {
            vk = vscale(z_k);
            ek = exp_fixed(vk - m);
        }
        if (lane_k) s_e[k] = ek;
        __syncthreads();
        if (tid == 0) {
            float E = 0.0f;
            s_E[0] = 0.0f;
            for (int i = 0; i < K; ++i) {
                E = E + s_e[i];
                s_E[i + 1] = E;
            }
        }
        __syncthreads();
        Z = s_E[K];
        int n_p = K, n_m = K;
        if ((rp.flags & SS_TOPP) && rp.top_p < 1.0f) {
            const float thr = rp.top_p * Z;
            n_p = block_count(k < K && s_E[k] < thr, s_redi);
        }
        if ((rp.flags & SS_MINP) && rp.min_p > 0.0f) {
            const float L = log_fixed(rp.min_p);
            n_m = block_count(k < K && (vk - m) >= L, s_redi);
        }
        n = min(n_p, n_m);
        En = s_E[n];
        uint32_t c1, c2;
        if (P.mode == MODE_VERIFY) {
            c1 = (uint32_t)b;
            c2 = (uint32_t)(row - b * P.rows_per_req);
        } else {
            c1 = (uint32_t)row;
            c2 = 0u;
        }
        const ss_rng rg = *P.rng;
        float s = 0.0f;
        const bool cand = k < n;
        if (cand) s = vk + gumbel_noise(rg.seed, rg.offset, (uint32_t)id_k, c1, c2);
        token = block_argmax(s, id_k, cand, s_redf, s_redi);
    }

    if (P.mode == MODE_SAMPLE) {
        if (tid == 0) {
            P.tokens[row] = token;
            if (P.status) P.status[row] = status;
            if (P.kept) P.kept[row] = live ? n : 0;
            if (P.mass) P.mass[row] = live ? (rp.greedy ? 1.0f : En / Z) : 0.0f;
        }
        if (lane_k) {
            if (P.topk_ids) P.topk_ids[(int64_t)row * KMAX + k] = (status != SS_ROW_INVALID && k < K) ? id_k : -1;
            if (P.probs) {
                float pk = 0.0f;
                if (live) pk = rp.greedy ? (k == 0 ? 1.0f : 0.0f) : (k < K ? ek / Z : 0.0f);
                P.probs[(int64_t)row * KMAX + k] = pk;
            }
        }
    } else {   // MODE_VERIFY
        RowRec* rec = P.recs + row;
        if (lane_k) {
            rec->ids[k] = (status != SS_ROW_INVALID && k < K) ? id_k : -1;
            rec->v[k] = vk;
            rec->p[k] = (live && !rp.greedy && k < n) ? ek / En : 0.0f;
        }
        if (tid == 0) {
            rec->n = live ? n : 0;
            rec->K = K;
            rec->token = token;
            rec->status = status;
            rec->greedy = rp.greedy;
        }
    }
}

}  // namespace ssd
