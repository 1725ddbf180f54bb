// Dense speculative verification: the target distribution p_j is the
// softmax of v = z/T over the whole vocabulary (no candidate bound, no
// truncation), draft probabilities q_j are read as whole rows (or are
// absent: then q counts as 1 at the draft token and the recovered token is
// drawn from p without it), as in the rejection and recovery kernels of the
// decoding notes ("Rejection Sampler").  The residual max(0, p - q) is
// sampled by a Gumbel-max on its logarithm (the notes' exponential race).
//
// Three fixed-grid launches:
//   dense_stats    one workgroup per (target row, 8192-token tile): the
//                  tile's best canonical logit as an (value, lower id) key
//                  and, for stochastic rows, sum exp(v - m_t) at the tile's
//                  own maximum m_t.  Workgroup 0 takes the step's copy of
//                  the Philox state and advances it.
//   dense_draw     one workgroup per (request, tile): every workgroup of a
//                  request combines the partials into m and Z per position
//                  (Z = sum_t s_t exp(m_t - m)) and walks the drafts
//                  (acceptance u q(d) <= p(d)); the one row that needs a
//                  draw over the whole vocabulary (the first rejection's
//                  residual, or the bonus row when every draft is accepted)
//                  is then processed tile by tile: best (ln r_i + g_i) or
//                  best (v_i + g_i) per tile.
//   dense_finish   one wave per request: merges the tile bests and writes
//                  the accepted prefix and the drawn token.
// Only the row that is drawn from is read twice; the others once.
#pragma once

#include "ss_stage2.h"

namespace ssd {

constexpr int DN_TILE = 8192;                     // tokens per tile workgroup
constexpr int DN_THREADS = 256;
constexpr int DN_EPT = DN_TILE / DN_THREADS;      // 32 tokens per thread
constexpr int DN_WAVES = DN_THREADS / WAVE;

// decision of one request, written by the draw workgroup of tile 0
struct DenseDec {
    int emitted;   // accepted drafts
    int token;     // final token when no draw is needed (-1: none)
    int status;
    int jdraw;     // row drawn from (-1: none)
    int mode;      // 1: residual of a rejection, 2: bonus
    int pad[3];
};

struct DenseParams {
    const void* target;
    int dtype, B, G, V, Zt;
    int64_t ld;
    int aligned16;
    const ss_req* req;
    ss_rng* rng;
    ss_rng* rng_snap;
    uint64_t rng_advance;
    const int32_t* cu_num_draft;
    const int32_t* draft_ids;
    const float* draft_probs;   // [B, G, V] or null
    uint64_t* part_k;           // [rows, Zt] best (value, id) key of the tile
    float* part_s;              // [rows, Zt] sum exp(v - m_t)
    uint64_t* draw_k;           // [B, Zt] best draw key of the tile
    DenseDec* dec;              // [B]
    int32_t* out_tokens;        // [B, G+1]
    int32_t* out_n_emit;
    int32_t* out_status;
};

constexpr uint32_t DN_PROCESSING = SS_GRAMMAR | SS_REP | SS_FREQPRES | SS_BIAS | SS_DRAFT_HIST;

// A request's mode: -1 invalid, 0 stochastic, 1 greedy; and its draft count.
__device__ __forceinline__ int dense_request(const DenseParams& D, int b, int& Gb) {
    const ss_req r = D.req[b];
    int mode = (r.flags & SS_GREEDY) ? 1 : 0;
    if (r.flags & DN_PROCESSING) mode = -1;
    const float T = r.temperature;
    if (mode == 0) {
        if (T != T) mode = -1;
        else if (T <= 0.0f) mode = 1;
        else if (T == bitsf(F32_PINF_BITS)) mode = -1;
    }
    Gb = D.G;
    if (D.cu_num_draft) {
        const int hi = D.cu_num_draft[b];
        const int lo = b > 0 ? D.cu_num_draft[b - 1] : 0;
        if (hi - lo < 0 || hi - lo > D.G) mode = -1;
        else Gb = hi - lo;
    }
    return mode;
}

// v = z/T clamped to the finite range; -inf stays -inf.
__device__ __forceinline__ float dense_v(float zc, float invT) {
    const float FMAX = bitsf(F32_MAX_BITS);
    float v = zc * invT;
    v = v > FMAX ? FMAX : v;
    v = v < -FMAX ? -FMAX : v;
    return zc == bitsf(F32_NINF_BITS) ? zc : v;
}

using dn_u32x4 = uint32_t __attribute__((ext_vector_type(4)));

// NaN -> -inf, +inf -> FLT_MAX (two min/max); -0 stays -0, which equals +0
// in every comparison, sum and exp here (only a key built from the value
// must add +0 first).
__device__ __forceinline__ float dense_canon(float x) {
    return fminf(fmaxf(x, bitsf(F32_NINF_BITS)), bitsf(F32_MAX_BITS));
}

// Canonical logits (dense_canon) of this thread's 32 tokens of tile `tile`
// (absent tokens read as -inf): element i is token dense_id(tile, i).
template <int DT>
__device__ __forceinline__ void dense_load(const DenseParams& D, int64_t row, int tile, float (&z)[DN_EPT]) {
    constexpr int EPC = DT == SS_BF16 ? 8 : 4;   // tokens per 16-byte chunk
    constexpr int NC = DN_EPT / EPC;
    const int base = tile * DN_TILE;
    const int nvalid = min(DN_TILE, D.V - base);
    const char* rowp = (const char*)D.target + (row * D.ld + base) * (DT == SS_BF16 ? 2 : 4);
    const int tid = threadIdx.x;
    if (nvalid == DN_TILE && D.aligned16) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const dn_u32x4 w = __builtin_nontemporal_load(gmem((const dn_u32x4*)rowp) + c * DN_THREADS + tid);
            const uint32_t d[4] = {w[0], w[1], w[2], w[3]};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (DT == SS_BF16) {
                    z[c * EPC + 2 * k] = dense_canon(bitsf(d[k] << 16));
                    z[c * EPC + 2 * k + 1] = dense_canon(bitsf(d[k] & 0xFFFF0000u));
                } else {
                    z[c * EPC + k] = dense_canon(bitsf(d[k]));
                }
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int k = 0; k < EPC; ++k) {
                const int e = (c * DN_THREADS + tid) * EPC + k;
                float x = bitsf(0x7FC00000u);
                if (e < nvalid) {
                    if constexpr (DT == SS_BF16) x = bitsf((uint32_t)gmem((const uint16_t*)rowp)[e] << 16);
                    else x = gmem((const float*)rowp)[e];
                }
                z[c * EPC + k] = dense_canon(x);
            }
    }
}

// token id of this thread's element i of tile `tile`
template <int DT>
__device__ __forceinline__ int dense_id(int tile, int i) {
    constexpr int EPC = DT == SS_BF16 ? 8 : 4;
    return tile * DN_TILE + ((i / EPC) * DN_THREADS + (int)threadIdx.x) * EPC + (i % EPC);
}

// (value, lower id first) key; -0 counts as +0 (s is never NaN)
__device__ __forceinline__ uint64_t dense_key(float s, int id) {
    return ((uint64_t)ord32(s + 0.0f) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}
__device__ __forceinline__ int dense_key_id(uint64_t k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }
__device__ __forceinline__ float dense_key_val(uint64_t k) { return unord32((uint32_t)(k >> 32)); }

// Butterfly reductions over the wave (distances 32, 16, .., 1; every lane
// ends with the result), exchanging through DPP and the row-swap permutes
// rather than the LDS crossbar.
template <int O = 32>
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
    const uint64_t x = xor_lane64<O>(k);
    k = x > k ? x : k;
    if constexpr (O > 1) return wave_max_u64<O / 2>(k);
    else return k;
}
template <int O = 32>
__device__ __forceinline__ float wave_max_f(float x) {
    x = fmaxf(x, __uint_as_float(xor_lane<O>(__float_as_uint(x))));
    if constexpr (O > 1) return wave_max_f<O / 2>(x);
    else return x;
}
template <int O = 32>
__device__ __forceinline__ float wave_sum_f(float x) {
    x += __uint_as_float(xor_lane<O>(__float_as_uint(x)));
    if constexpr (O > 1) return wave_sum_f<O / 2>(x);
    else return x;
}

template <int DT>
__global__ __launch_bounds__(DN_THREADS) void dense_stats_kernel(DenseParams D) {
    __shared__ uint64_t s_key[DN_WAVES];
    __shared__ float s_m[DN_WAVES], s_s[DN_WAVES];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / WAVE;
    if (blockIdx.x == 0 && tid == 0) {   // the step's copy of the generator state
        const ss_rng r = *D.rng;
        *D.rng_snap = r;
        if (D.rng_advance) D.rng->offset = r.offset + D.rng_advance;
    }
    const int row = (int)blockIdx.x / D.Zt;
    const int tile = (int)blockIdx.x - row * D.Zt;
    const int b = row / (D.G + 1), j = row - b * (D.G + 1);
    int Gb;
    const int mode = dense_request(D, b, Gb);
    if (mode < 0 || j > Gb) return;   // block-uniform
    const float NINF = bitsf(F32_NINF_BITS), FMAX = bitsf(F32_MAX_BITS);
    float z[DN_EPT];
    dense_load<DT>(D, row, tile, z);   // canonical, absent tokens -inf
    // the thread's best canonical value (the max of the canonical values)
    float zt = NINF;
#pragma unroll
    for (int i = 0; i < DN_EPT; ++i) zt = fmaxf(zt, z[i]);
    uint64_t key;
    if (mode == 1) {
        // greedy: the lowest id holding it (ids grow with i within a thread)
        int first = DN_EPT - 1;
#pragma unroll
        for (int i = DN_EPT - 1; i >= 0; --i) first = z[i] == zt ? i : first;
        int id = 0;
#pragma unroll
        for (int i = 0; i < DN_EPT; ++i) id = i == first ? dense_id<DT>(tile, i) : id;
        key = dense_key(zt, id);
    } else {
        key = dense_key(zt, 0);   // stochastic rows need the value only
    }
    key = wave_max_u64(key);
    // stochastic rows: sum exp(v - m) at this thread's maximum m, rescaled to
    // the tile's below.  The terms only feed the sum Z, so they take the
    // hardware exp2 on z (a/ln 2) - m/ln 2 whenever no z/T leaves the
    // finite range and m is far from -FLT_MAX (then the clamps of v change
    // no term); otherwise the exact form.
    float m = NINF, s = 0.0f;
    if (mode == 0) {
        const float invT = 1.0f / D.req[b].temperature;
        m = dense_v(zt, invT);
        if (m != NINF) {
            const float big = zt * invT;
            if (big <= FMAX && m > -0x1p127f) {
                const float a = invT * 0x1.715476p+0f, c = m * 0x1.715476p+0f;
#pragma unroll
                for (int i = 0; i < DN_EPT; ++i) s += __builtin_amdgcn_exp2f(__builtin_fmaf(z[i], a, -c));
            } else {
#pragma unroll
                for (int i = 0; i < DN_EPT; ++i) s += exp_fixed_nonpos(dense_v(z[i], invT) - m);
            }
        }
        const float wm = wave_max_f(m);
        s = (wm == NINF || m == NINF) ? 0.0f : s * exp_fixed_nonpos(m - wm);
        s = wave_sum_f(s);
        m = wm;
    }
    if (lane == 0) {
        s_key[wave] = key;
        s_m[wave] = m;
        s_s[wave] = s;
    }
    __syncthreads();
    if (tid == 0) {
        uint64_t k = s_key[0];
        float mt = s_m[0];
        for (int w = 1; w < DN_WAVES; ++w) {
            k = s_key[w] > k ? s_key[w] : k;
            mt = fmaxf(mt, s_m[w]);
        }
        float st = 0.0f;
        if (mt != NINF)
            for (int w = 0; w < DN_WAVES; ++w)
                st += s_m[w] == NINF ? 0.0f : s_s[w] * exp_fixed_nonpos(s_m[w] - mt);
        D.part_k[(int64_t)row * D.Zt + tile] = k;
        D.part_s[(int64_t)row * D.Zt + tile] = st;
    }
}

// m and Z of row `row` from its tile partials (wave-wide; every lane gets
// them), and its best key.  m_t is recomputed from the tile's best value.
__device__ __forceinline__ void dense_row_stats(const DenseParams& D, int64_t row, float invT, bool stoch,
                                                uint64_t& best, float& m, float& Z) {
    const int lane = lane_id();
    uint64_t k = 0;
    for (int t = lane; t < D.Zt; t += WAVE) {
        const uint64_t x = D.part_k[row * D.Zt + t];
        k = x > k ? x : k;
    }
    best = wave_max_u64(k);
    m = bitsf(F32_NINF_BITS);
    Z = 0.0f;
    if (!stoch) return;
    m = dense_v(dense_key_val(best), invT);
    float acc = 0.0f;
    if (m != bitsf(F32_NINF_BITS)) {
        for (int t = lane; t < D.Zt; t += WAVE) {
            const float mt = dense_v(dense_key_val(D.part_k[row * D.Zt + t]), invT);
            const float st = D.part_s[row * D.Zt + t];
            acc += mt == bitsf(F32_NINF_BITS) ? 0.0f : st * exp_fixed_nonpos(mt - m);
        }
    }
    Z = wave_sum_f(acc);
}

template <int DT>
__global__ __launch_bounds__(DN_THREADS) void dense_draw_kernel(DenseParams D) {
    __shared__ DenseDec s_dec;
    __shared__ float s_mz[2];
    __shared__ uint64_t s_best[DN_WAVES];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / WAVE;
    const int b = (int)blockIdx.x / D.Zt;
    const int tile = (int)blockIdx.x - b * D.Zt;
    const ss_rng rg = *D.rng_snap;
    int Gb;
    const int mode = dense_request(D, b, Gb);
    const float T = D.req[b].temperature;
    const float invT = mode == 0 ? 1.0f / T : 1.0f;
    // every position's outcome in parallel (wave w: positions w, w + 4, ..),
    // then one thread walks them in order; every workgroup of the request
    // finds the same
    __shared__ int s_acc[SS_GAMMA_MAX + 1], s_top[SS_GAMMA_MAX + 1], s_masked[SS_GAMMA_MAX + 1];
    __shared__ float s_pm[SS_GAMMA_MAX + 1], s_pz[SS_GAMMA_MAX + 1];
    for (int j = wave; mode >= 0 && j <= Gb; j += DN_WAVES) {
        const int64_t row = (int64_t)b * (D.G + 1) + j;
        // the draft's logit and probability are requested with the partials
        const int d = j < Gb ? D.draft_ids[(int64_t)b * D.G + j] : -1;
        const bool din = (unsigned)d < (unsigned)D.V;
        const void* rp = (const char*)D.target + row * D.ld * (DT == SS_BF16 ? 2 : 4);
        float zd = 0.0f, qd = 0.0f;
        if (din && mode == 0) {
            if constexpr (DT == SS_BF16) zd = canon(bitsf((uint32_t)((const uint16_t*)rp)[d] << 16));
            else zd = canon(((const float*)rp)[d]);
            qd = D.draft_probs ? D.draft_probs[((int64_t)b * D.G + j) * D.V + d] : 1.0f;
        }
        uint64_t best;
        float m, Z;
        dense_row_stats(D, row, invT, mode == 0, best, m, Z);
        const int top = dense_key_id(best);
        const bool masked = dense_key_val(best) == bitsf(F32_NINF_BITS);
        int acc;
        if (mode == 1) {
            acc = j < Gb && d == top;
        } else if (j < Gb) {
            const float pd = din ? exp_fixed_nonpos(dense_v(zd, invT) - m) / Z : 0.0f;
            const float u = unit_open(philox_w0(rg.seed, rg.offset, 0u, (uint32_t)b, (1u << 24) | (uint32_t)j));
            acc = qd > 0.0f && u * qd <= pd;
        } else {
            acc = 0;
        }
        if (lane == 0) {
            s_acc[j] = acc;
            s_top[j] = top;
            s_masked[j] = masked;
            s_pm[j] = m;
            s_pz[j] = Z;
        }
    }
    __syncthreads();
    if (tid == 0) {
        DenseDec dc{0, -1, SS_ROW_OK, -1, 0, {0, 0, 0}};
        float mdraw = 0.0f, Zdraw = 1.0f;
        if (mode < 0) dc.status = SS_ROW_INVALID;
        for (int j = 0; mode >= 0 && j <= Gb; ++j) {
            if (s_masked[j]) {
                dc.status = SS_ROW_ALL_MASKED;
                break;
            }
            if (s_acc[j]) {
                ++dc.emitted;
                continue;
            }
            if (mode == 1) {
                dc.token = s_top[j];
            } else {
                dc.jdraw = j;
                dc.mode = j == Gb ? 2 : 1;   // every draft accepted: the bonus from row Gb
                mdraw = s_pm[j];
                Zdraw = s_pz[j];
            }
            break;
        }
        s_dec = dc;
        s_mz[0] = mdraw;
        s_mz[1] = Zdraw;
    }
    __syncthreads();
    const DenseDec dc = s_dec;
    if (tile == 0 && tid == 0) D.dec[b] = dc;
    if (dc.jdraw < 0) return;   // block-uniform
    const int jd = dc.jdraw;
    const int64_t row = (int64_t)b * (D.G + 1) + jd;
    float z[DN_EPT];
    dense_load<DT>(D, row, tile, z);
    const float m = s_mz[0], Z = s_mz[1];
    const uint32_t c2 = dc.mode == 2 ? (uint32_t)Gb : ((2u << 24) | (uint32_t)jd);
    const int d = dc.mode == 1 ? D.draft_ids[(int64_t)b * D.G + jd] : -1;
    const float* q = (dc.mode == 1 && D.draft_probs) ? D.draft_probs + ((int64_t)b * D.G + jd) * D.V : nullptr;
    uint64_t key = 0;
    if (q) {
        // With draft probabilities about half the tokens have rho = p - q
        // > 0: those are queued per wave in LDS, and the logarithm and the
        // Gumbel noise are worked out over the queue in full rounds of 64
        // lanes.  Each candidate's arithmetic is the direct path's and the
        // keys are unique, so the maximum does not depend on the order.
        // (Without q every token but the draft is a candidate, and the
        // queue would only add work.)
        constexpr int QSLOTS = 8;   // token slots per queue fill
        __shared__ int s_qid[DN_WAVES][QSLOTS * WAVE];
        __shared__ float s_qx[DN_WAVES][QSLOTS * WAVE];
#pragma unroll
        for (int g = 0; g < DN_EPT; g += QSLOTS) {
            int n = 0;   // queue length (uniform)
#pragma unroll
            for (int i = g; i < g + QSLOTS; ++i) {
                const int id = dense_id<DT>(tile, i);
                float rho = 0.0f;
                if (id < D.V) rho = exp_fixed_nonpos(dense_v(z[i], invT) - m) / Z - q[id];
                const bool cand = rho > 0.0f;
                const uint64_t bal = __ballot(cand);
                if (cand) {
                    const int slot = n + lane_prefix(bal);
                    s_qid[wave][slot] = id;
                    s_qx[wave][slot] = rho;
                }
                n += __popcll(bal);
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
            for (int k = lane; k < n; k += WAVE) {
                const int id = s_qid[wave][k];
                const float sc = log_fixed(s_qx[wave][k]) +
                                 gumbel_noise(rg.seed, rg.offset, (uint32_t)id, (uint32_t)b, c2);
                const uint64_t kk = dense_key(sc, id);   // > 0 for every candidate
                key = kk > key ? kk : key;
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // read before the next fill
            __builtin_amdgcn_wave_barrier();
        }
    } else {
#pragma unroll
        for (int i = 0; i < DN_EPT; ++i) {
            const int id = dense_id<DT>(tile, i);
            if (id >= D.V) continue;
            const float v = dense_v(z[i], invT);
            float sc;
            if (dc.mode == 2) {
                sc = v + gumbel_noise(rg.seed, rg.offset, (uint32_t)id, (uint32_t)b, c2);
            } else {
                const float rho = id == d ? 0.0f : exp_fixed_nonpos(v - m) / Z;
                if (!(rho > 0.0f)) continue;
                sc = log_fixed(rho) + gumbel_noise(rg.seed, rg.offset, (uint32_t)id, (uint32_t)b, c2);
            }
            const uint64_t kk = dense_key(sc, id);   // > 0 for every candidate (sc is never NaN)
            key = kk > key ? kk : key;
        }
    }
    key = wave_max_u64(key);
    if (lane == 0) s_best[wave] = key;
    __syncthreads();
    if (tid == 0) {
        uint64_t k = s_best[0];
        for (int w = 1; w < DN_WAVES; ++w) k = s_best[w] > k ? s_best[w] : k;
        D.draw_k[(int64_t)b * D.Zt + tile] = k;
    }
}

// One wave per request: the accepted prefix, then the drawn token.
template <int DT>
__global__ __launch_bounds__(WAVE) void dense_finish_kernel(DenseParams D) {
    const int b = blockIdx.x;
    const int lane = lane_id();
    const DenseDec dc = D.dec[b];
    int token = dc.token;
    if (dc.jdraw >= 0) {
        uint64_t k = 0;
        for (int t = lane; t < D.Zt; t += WAVE) {
            const uint64_t x = D.draw_k[(int64_t)b * D.Zt + t];
            k = x > k ? x : k;
        }
        k = wave_max_u64(k);
        if (k != 0) {
            token = dense_key_id(k);
        } else {
            // p <= q at every token: draw from p, v_i + g_i over the row
            const ss_rng rg = *D.rng_snap;
            const int jd = dc.jdraw;
            const float invT = 1.0f / D.req[b].temperature;
            const uint32_t c2 = (2u << 24) | (uint32_t)jd;
            const char* rp = (const char*)D.target + ((int64_t)b * (D.G + 1) + jd) * D.ld * (DT == SS_BF16 ? 2 : 4);
            uint64_t best = 0;
            for (int i = lane; i < D.V; i += WAVE) {
                float zc;
                if constexpr (DT == SS_BF16) zc = canon(bitsf((uint32_t)((const uint16_t*)rp)[i] << 16));
                else zc = canon(((const float*)rp)[i]);
                const float s = dense_v(zc, invT) + gumbel_noise(rg.seed, rg.offset, (uint32_t)i, (uint32_t)b, c2);
                const uint64_t x = dense_key(s, i);
                best = x > best ? x : best;
            }
            token = dense_key_id(wave_max_u64(best));
        }
    }
    if (lane == 0) {
        int32_t* out = D.out_tokens + (int64_t)b * (D.G + 1);
        int n = 0;
        if (dc.status != SS_ROW_INVALID) {
            for (; n < dc.emitted; ++n) out[n] = D.draft_ids[(int64_t)b * D.G + n];
            if (dc.status == SS_ROW_OK) out[n++] = token;
        }
        for (int j = n; j <= D.G; ++j) out[j] = -1;
        D.out_n_emit[b] = n;
        if (D.out_status) D.out_status[b] = dc.status;
    }
}

}  // namespace ssd
