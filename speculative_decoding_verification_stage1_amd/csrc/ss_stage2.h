// Stage 2 (SonicSampler section 3.2 and Fig. 1, stage 2) for one row: the
// row's Z_v tile lists are re-indexed to global token ids and merged with
// bitonic merge networks into the row's 128 best tokens; then the fused
// epilogue runs: temperature, softmax weights, top-p / min-p truncation
// and Gumbel-max selection (section 3.1 "Probability truncation",
// "Sampling").
//
// One workgroup per row.  Each wave folds a share of the row's tile lists
// into one sorted list held in registers (two keys per lane: ranks lane and
// lane + 64), with bitonic merge networks built from cross-lane shuffles;
// wave 0 then folds the per-wave lists and the listed tokens and runs the
// epilogue, so the whole stage needs two workgroup barriers.
//
// Tokens named by an active penalty or bias list never enter the tiles;
// Stage 2 computes their processed logits directly (gather + the list
// arithmetic in list order) and merges them as one more sorted list.
//
// Merge key (64-bit, larger = better): ord32(z) << 32 | (0xFFFFFFFF - id).
#pragma once

#include "ss_stage1.h"
#include "ss_wavesort.h"

namespace ssd {

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

struct Stage2Params {
    Stage1Params s1;
    const ss_rng* rng;
    const uint64_t* listed;   // [rows][128] sorted merge keys of listed tokens
    int mode;
    int topk_k;
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
    const int32_t* cu_num_draft;   // optional [B] inclusive cumulative draft counts
    int32_t* v_tokens;
    int32_t* v_n_emit;
    int32_t* v_status;
    uint32_t* arrive;   // verification decided in Stage 2: one 64-bit word per request (else null)
    // top-k
    float* topk_vals;
};

struct S2Shared {
    uint64_t wl[4][2][WAVE];   // per-wave folded lists (lo, hi)
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
// bias_head: this lane's entry lane of the request's bias values when the
// caller requested it early (NaN-free check), else read here.
// rq_pre: the request record's eight words when the caller requested them
// early, else read here.
__device__ inline RowParams row_params(const Stage1Params& P, int b, const float* bias_head = nullptr,
                                       const uint32_t* rq_pre = nullptr) {
    RowParams rp{};
    if (!P.req) {   // plain top-k: no processing
        rp.valid = 1;
        rp.greedy = 1;
        rp.K = min(KMAX, P.V);
        return rp;
    }
    ss_req r;
    if (rq_pre) {
        static_assert(sizeof(ss_req) == 8 * sizeof(uint32_t), "request record");
        __builtin_memcpy(&r, rq_pre, sizeof(r));
    } else {
        r = P.req[b];
    }
    const uint32_t f = r.flags;
    rp.flags = f;
    rp.temperature = r.temperature;
    rp.top_p = r.top_p;
    rp.min_p = r.min_p;
    rp.rep = r.rep_penalty;
    rp.freq = r.freq_penalty;
    rp.pres = r.pres_penalty;
    bool ok = true;
    if ((int)r.n_prior > P.aux.prior_stride || (int)r.n_bias > P.aux.bias_stride || r.n_prior > SS_PRIOR_MAX ||
        r.n_bias > SS_BIAS_MAX)
        ok = false;
    if ((f & SS_GRAMMAR) && !P.aux.bitmask) ok = false;
    if ((f & (SS_REP | SS_FREQPRES)) && r.n_prior > 0 && (!P.aux.prior_ids || !P.aux.prior_cnt)) ok = false;
    if ((f & SS_BIAS) && r.n_bias > 0 && (!P.aux.bias_ids || !P.aux.bias_val)) ok = false;
    if ((f & SS_REP) && !(finitef(r.rep_penalty) && r.rep_penalty > 0.0f)) ok = false;
    if ((f & SS_FREQPRES) && !(finitef(r.freq_penalty) && finitef(r.pres_penalty))) ok = false;
    if (ok && (f & SS_BIAS)) {   // every bias value finite: lanes check in parallel
        const auto bv = gmem(P.aux.bias_val + (int64_t)b * P.aux.bias_stride);
        bool bad = false;
        int j0 = 0;
        if (bias_head) {
            bad = lane_id() < (int)r.n_bias && !finitef(*bias_head);
            j0 = WAVE;
        }
        for (int j = j0 + lane_id(); j < (int)r.n_bias; j += WAVE) bad |= !finitef(bv[j]);
        ok = __ballot(bad) == 0ull;
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

using WL64 = WList<uint64_t>;

// Lists up to this length are ranked by one wave of the Stage-1 launch
// (staged in that wave's LDS area); longer ones by listed_long_kernel.
constexpr int LIST_SHORT = 256;

// The row's side lists, staged in LDS by the listed-token workgroup.
struct S2Lists {
    int32_t pid[LIST_SHORT + SS_GAMMA_MAX];   // prior entries, then entries for earlier drafts
    int32_t pct[LIST_SHORT + SS_GAMMA_MAX];
    int32_t bid[LIST_SHORT];
    float bval[LIST_SHORT];
};

// Open-addressing table of the ids named by a row's lists (at most KMAX
// entries, so the table is never more than half full): the id, the
// smallest combined position (prior entries first, then bias entries)
// naming it, and its live prior entries (low 16 bits) and bias entries
// (high 16 bits).
constexpr int LIST_HASH = 256;
struct ListedTable {
    uint32_t id[LIST_HASH];   // ~0: empty
    uint32_t first[LIST_HASH];
    uint32_t cnt[LIST_HASH];
};

__device__ __forceinline__ void listed_table_clear(ListedTable& T) {
    const uint4 ones{~0u, ~0u, ~0u, ~0u}, zero{0u, 0u, 0u, 0u};
    for (int i = lane_id(); i < LIST_HASH / 4; i += WAVE) {
        ((uint4*)T.id)[i] = ones;
        ((uint4*)T.first)[i] = ones;
        ((uint4*)T.cnt)[i] = zero;
    }
}

// Listed tokens: exact processed logits of the first
// valid entry of every id named by an active list, sorted; at most KMAX
// combined entries (two per lane).
//
// Each valid entry enters its id into the row's table, which gives every
// entry its id's first position and its number of prior and bias entries;
// only the first entry of an id makes a key.  The repetition penalty is the
// same map for every entry, so m matching entries apply it m times.
// Frequency/presence and bias differ per entry and must be applied in list
// order; with one matching entry (the usual case) that is the entry's own
// subtraction / addition, and tokens with several entries take a sequential
// walk of the list.  The logits at the listed ids are requested before the
// table is built, so the table hides their latency.
template <int DT>
__device__ __forceinline__ WL64 listed_list(const Stage1Params& P, const RowParams& rp, int row, int np, int nb,
                                            const S2Lists& L, ListedTable& T) {
    const int lane = lane_id();
    const int ncomb = np + nb;
    const bool grammar = (rp.flags & SS_GRAMMAR) != 0;
    const bool do_rep = (rp.flags & SS_REP) != 0;
    const bool do_fp = (rp.flags & SS_FREQPRES) != 0;
    const bool do_bias = (rp.flags & SS_BIAS) != 0;
    int t[2], id[2];
    bool ok[2];
    uint32_t raw[2], word[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        t[h] = h * WAVE + lane;
        id[h] = -1;
        ok[h] = false;
        if (t[h] < np) {
            id[h] = L.pid[t[h]];
            ok[h] = L.pct[t[h]] >= 1 && id[h] >= 0 && id[h] < P.V;
        } else if (t[h] < ncomb) {
            id[h] = L.bid[t[h] - np];
            ok[h] = id[h] >= 0 && id[h] < P.V;
        }
        const int ic = ok[h] ? id[h] : 0;   // every lane loads, from column 0 if it has no entry
        if (DT == SS_BF16) raw[h] = ((const uint16_t*)P.logits)[(int64_t)row * P.ld + ic];
        else raw[h] = __float_as_uint(((const float*)P.logits)[(int64_t)row * P.ld + ic]);
        word[h] = grammar ? P.aux.bitmask[(int64_t)row * P.aux.bitmask_stride + (ic >> 5)] : ~0u;
    }
    uint32_t slot[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        slot[h] = 0;
        if (ok[h]) {
            uint32_t s = ((uint32_t)id[h] * 0x9E3779B1u) >> 24;
            for (;;) {   // ends: fewer entries than slots
                const uint32_t o = atomicCAS(&T.id[s], ~0u, (uint32_t)id[h]);
                if (o == ~0u || o == (uint32_t)id[h]) break;
                s = (s + 1) & (LIST_HASH - 1);
            }
            slot[h] = s;
            atomicMin(&T.first[s], (uint32_t)t[h]);
            atomicAdd(&T.cnt[s], t[h] < np ? 1u : 0x10000u);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    uint64_t key[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const bool lead = ok[h] && T.first[slot[h]] == (uint32_t)t[h];
        const uint32_t c = T.cnt[slot[h]];
        const int mp = (int)(c & 0xFFFFu), mb = (int)(c >> 16);
        float zz = DT == SS_BF16 ? widen_bf16((uint16_t)raw[h]) : __uint_as_float(raw[h]);
        if (!((word[h] >> (id[h] & 31)) & 1u)) zz = bitsf(F32_NINF_BITS);
        if (lead) {
            if (do_rep)
                for (int r = 0; r < mp; ++r) zz = (zz > 0.0f) ? zz / rp.rep : zz * rp.rep;
            if (do_fp) {
                if (mp == 1) {   // the entry itself (prior entries come first)
                    zz = zz - ((float)L.pct[t[h]] * rp.freq + rp.pres);
                } else if (mp > 1) {
                    for (int u = 0; u < np; ++u)
                        if (L.pct[u] >= 1 && L.pid[u] == id[h]) zz = zz - ((float)L.pct[u] * rp.freq + rp.pres);
                }
            }
            if (do_bias) {
                if (mb == 1 && t[h] >= np) zz = zz + L.bval[t[h] - np];   // the entry itself
                else if (mb >= 1)
                    for (int u = 0; u < nb; ++u)
                        if (L.bid[u] == id[h]) zz = zz + L.bval[u];
            }
        }
        key[h] = lead ? (((uint64_t)ord32(canon(zz)) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id[h])) : 0ull;
    }
    return wave_sort128(WL64{key[0], key[1]});
}

// ---- listed tokens by sorting: the row's entries (prior entries, then the
// earlier drafts of a verification row, then bias entries) become keys
// id << 16 | position; sorted, the entries of one token lie together in
// list order, and the entry that starts a token walks them.  Used by one
// wave for rows with more than 128 entries, and by listed_long_kernel (one
// workgroup per row) for lists longer than LIST_SHORT. ----

// Entry key of combined position i (~0: the entry names no token).
__device__ __forceinline__ uint64_t listed_entry_key(const Stage1Params& P, int b, int i, int np, int nh) {
    int id;
    bool ok;
    if (i < np) {
        const int64_t o = (int64_t)b * P.aux.prior_stride + i;
        id = gmem(P.aux.prior_ids)[o];
        ok = gmem(P.aux.prior_cnt)[o] >= 1;
    } else if (i < np + nh) {
        id = gmem(P.draft_ids)[(int64_t)b * (P.rows_per_req - 1) + (i - np)];
        ok = true;
    } else {
        id = gmem(P.aux.bias_ids)[(int64_t)b * P.aux.bias_stride + (i - np - nh)];
        ok = true;
    }
    return ok && id >= 0 && id < P.V ? ((uint64_t)(uint32_t)id << 16) | (uint64_t)i : ~0ull;
}

// The merge key of the token whose entries start at sorted position i of
// k[0, ns), or 0 if position i does not start one: its logit (grammar
// mask applied), the repetition map once per live prior entry, then each
// prior entry's frequency/presence subtraction in list order, then each
// bias addition; the earlier drafts add to the count of the token's first
// live prior entry, or form one appended entry.
template <int DT, typename KP>
__device__ __forceinline__ uint64_t listed_token_key(const Stage1Params& P, const RowParams& rp, int row, int b,
                                                     KP k, int ns, int i, int np, int nh) {
    const uint64_t e = k[i];
    if (e == ~0ull) return 0ull;
    const uint32_t id = (uint32_t)(e >> 16);
    if (i > 0 && k[i - 1] != ~0ull && (uint32_t)(k[i - 1] >> 16) == id) return 0ull;   // not the first
    int end = i + 1;
    while (end < ns && k[end] != ~0ull && (uint32_t)(k[end] >> 16) == id) ++end;
    int first_prior = -1, ndraft = 0;
    for (int t = i; t < end; ++t) {
        const int pos = (int)(k[t] & 0xFFFFu);
        if (pos < np) {
            if (first_prior < 0) first_prior = pos;
        } else if (pos < np + nh) {
            ++ndraft;
        }
    }
    const bool appended = first_prior < 0 && ndraft > 0;
    const int64_t po = (int64_t)b * P.aux.prior_stride, bo = (int64_t)b * P.aux.bias_stride;
    float z;
    if (DT == SS_BF16) z = widen_bf16(((const uint16_t*)P.logits)[(int64_t)row * P.ld + id]);
    else z = ((const float*)P.logits)[(int64_t)row * P.ld + id];
    if ((rp.flags & SS_GRAMMAR) &&
        !((P.aux.bitmask[(int64_t)row * P.aux.bitmask_stride + (id >> 5)] >> (id & 31)) & 1u))
        z = bitsf(F32_NINF_BITS);
    if (rp.flags & SS_REP) {
        for (int t = i; t < end; ++t)
            if ((int)(k[t] & 0xFFFFu) < np) z = (z > 0.0f) ? z / rp.rep : z * rp.rep;
        if (appended) z = (z > 0.0f) ? z / rp.rep : z * rp.rep;
    }
    if (rp.flags & SS_FREQPRES) {
        for (int t = i; t < end; ++t) {
            const int pos = (int)(k[t] & 0xFFFFu);
            if (pos >= np) continue;
            const int c = gmem(P.aux.prior_cnt)[po + pos] + (pos == first_prior ? ndraft : 0);
            z = z - ((float)c * rp.freq + rp.pres);
        }
        if (appended) z = z - ((float)ndraft * rp.freq + rp.pres);
    }
    if (rp.flags & SS_BIAS)
        for (int t = i; t < end; ++t) {
            const int pos = (int)(k[t] & 0xFFFFu);
            if (pos >= np + nh) z = z + gmem(P.aux.bias_val)[bo + (pos - np - nh)];
        }
    return ((uint64_t)ord32(canon(z)) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}

// Entries of a row with more than 128 in one wave's area (keys of up to
// 2 * LIST_SHORT + SS_GAMMA_MAX entries, padded to a power of two).
constexpr int LW_CAP = 1024;
static_assert(2 * LIST_SHORT + SS_GAMMA_MAX <= LW_CAP, "wave sort capacity");

// One wave's LDS area in the listed-token workgroups: the staged lists, or
// the entry keys of the sorting form.
struct ListedStage {
    S2Lists lists;
    ListedTable table;
};
union ListedArea {
    ListedStage st;
    uint64_t keys[LW_CAP];
};
static_assert(sizeof(ListedStage) <= sizeof(uint64_t) * LW_CAP, "listed staging area");

// The sorting form in one wave: out[row] = the best 128 listed tokens.
// (Made a separate, not inlined function, c2's Stage 1 took twice as
// long, although c2's rows never call it.)
template <int DT>
__device__ __forceinline__ void listed_row_sorted(const Stage1Params& P, const RowParams& rp, uint64_t* out,
                                                  int row, int b, int np, int nh, int nb, uint64_t* k) {
    const int lane = lane_id();
    const int n = np + nh + nb;
    int ns = 2 * KMAX;
    while (ns < n) ns <<= 1;
    for (int i = lane; i < ns; i += WAVE) k[i] = i < n ? listed_entry_key(P, b, i, np, nh) : ~0ull;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    for (int size = 2; size <= ns; size <<= 1)   // ascending bitonic sort
        for (int j = size >> 1; j > 0; j >>= 1) {
            for (int i = lane; i < ns / 2; i += WAVE) {
                const int lo = ((i & ~(j - 1)) << 1) | (i & (j - 1));
                const int hi = lo + j;
                const uint64_t a = k[lo], c = k[hi];
                if ((a > c) == ((lo & size) == 0)) {
                    k[lo] = c;
                    k[hi] = a;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }
    constexpr int PER = LW_CAP / WAVE;
    uint64_t res[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int i = lane + q * WAVE;
        res[q] = i < ns ? listed_token_key<DT>(P, rp, row, b, k, ns, i, np, nh) : 0ull;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int q = 0; q < PER; ++q)
        if (lane + q * WAVE < ns) k[lane + q * WAVE] = res[q];
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    WL64 acc{0ull, 0ull};
    for (int c0 = 0; c0 < ns; c0 += KMAX) {
        const WL64 l = wave_sort128(WL64{k[c0 + lane], k[c0 + lane + WAVE]});
        acc = c0 == 0 ? l : wave_merge(acc, l);
    }
    out[(int64_t)row * KMAX + lane] = acc.lo;
    out[(int64_t)row * KMAX + lane + WAVE] = acc.hi;
}

// One workgroup of the Stage-1 launch per row computes the row's listed
// tokens (wave 0) and stores the best 128 as merge keys; it runs alongside
// the tile workgroups, so Stage 2 only has to load one more sorted list.
// One wave computes row `row`'s listed tokens: its lists are staged in the
// wave's own LDS area, then ranked as exact keys (list order arithmetic).
template <int DT>
__device__ __forceinline__ void listed_row_wave(const Stage1Params& P, uint64_t* out, int row, ListedArea& area) {
    S2Lists& lists = area.st.lists;
    const int b = __builtin_amdgcn_readfirstlane(div_uniform(row, P.rows_per_req));
    const RowParams rp = row_params(P, b);
    int np = rp.valid ? rp.n_prior : 0;
    const int nb = rp.valid ? rp.n_bias : 0;
    const int nh = rp.valid ? draft_hist_len(P, rp.flags, row) : 0;
    if (np + nb + nh == 0) return;   // wave-uniform; Stage 2 skips rows without lists
    if (np > LIST_SHORT || nb > LIST_SHORT) return;   // ranked by listed_long_kernel
    if (np + nb + nh > KMAX) {   // more than one pass of the scan below: sort instead
        // this form can outlast the tiles: ahead of the tile waves (priority
        // 1; the other listed-token waves keep 0)
        __builtin_amdgcn_s_setprio(2);
        listed_row_sorted<DT>(P, rp, out, row, b, np, nh, nb, area.keys);
        return;
    }
    const auto pid = gmem(P.aux.prior_ids + (int64_t)b * P.aux.prior_stride);
    const auto pct = gmem(P.aux.prior_cnt + (int64_t)b * P.aux.prior_stride);
    const auto bid = gmem(P.aux.bias_ids + (int64_t)b * P.aux.bias_stride);
    const auto bvl = gmem(P.aux.bias_val + (int64_t)b * P.aux.bias_stride);
    const int lane = lane_id();
    listed_table_clear(area.st.table);
    for (int u = lane; u < np; u += WAVE) {
        lists.pid[u] = pid[u];
        lists.pct[u] = pct[u];
    }
    for (int u = lane; u < nb; u += WAVE) {
        lists.bid[u] = bid[u];
        lists.bval[u] = bvl[u];
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (nh > 0) {
        // the drafts before this position join the history in order: one
        // more occurrence on the first live entry of the id, else a new
        // entry for it
        const int dl = lane < nh ? gmem(P.draft_ids)[(int64_t)b * (P.rows_per_req - 1) + lane] : -1;
        for (int i = 0; i < nh; ++i) {   // uniform
            const int dv = __builtin_amdgcn_readlane(dl, i);
            if (dv < 0 || dv >= P.V) continue;
            int hit = -1;
            for (int k0 = 0; k0 < np && hit < 0; k0 += WAVE) {
                const int k = k0 + lane;
                const uint64_t m = __ballot(k < np && lists.pid[k] == dv && lists.pct[k] >= 1);
                if (m) hit = k0 + __builtin_ctzll(m);
            }
            if (lane == 0) {
                if (hit >= 0) {
                    lists.pct[hit] += 1;
                } else {
                    lists.pid[np] = dv;
                    lists.pct[np] = 1;
                }
            }
            if (hit < 0) ++np;
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }
    }
    const WL64 l = listed_list<DT>(P, rp, row, np, nb, lists, area.st.table);
    out[(int64_t)row * KMAX + lane] = l.lo;
    out[(int64_t)row * KMAX + lane + WAVE] = l.hi;
}

constexpr int S2_THREADS = 256;
constexpr int S2_WAVES = S2_THREADS / WAVE;
constexpr int S2_PREFETCH = 4;   // tile lists per wave requested up front

// The row's Stage-1 lists, requested before anything else in Stage 2.
template <int DT>
struct RowLoads {
    typename S1Traits<DT>::Key pre_lo[S2_PREFETCH], pre_hi[S2_PREFETCH];
    WL64 listed;
    float bias_head;   // bias value `lane` of the request (validation)
    uint32_t rq[8];    // the request record
};
template <int DT>
__device__ __forceinline__ void row_loads(const Stage2Params& F, int row, RowLoads<DT>& L) {
    using Key = typename S1Traits<DT>::Key;
    const Stage1Params& P = F.s1;
    const int lane = lane_id();
    const int wave = threadIdx.x / WAVE;
    // the request record and the bias values first: the row's parameters
    // are worked out while the lists arrive
    if (P.req) {
        const auto rq = gmem((const uint32_t*)(P.req + div_uniform(row, P.rows_per_req)));
#pragma unroll
        for (int i = 0; i < 8; ++i) L.rq[i] = rq[i];
    }
    // bias value `lane` (zero past the stride or without values)
    {
        const int b = div_uniform(row, P.rows_per_req);
        const auto bv = buf_view(P.aux.bias_val + (P.aux.bias_val ? (int64_t)b * P.aux.bias_stride : 0),
                                 P.aux.bias_val ? (uint32_t)P.aux.bias_stride * 4u : 0u);
        L.bias_head = __uint_as_float(buf_u32(bv, (uint32_t)lane * 4u));
    }
    // the tile lists: a fixed run of loads over the row's lists (tiles past
    // Zv read as key 0, no token)
    const auto sv = buf_view((const Key*)P.scratch + (int64_t)row * P.Zv * KMAX,
                             (uint32_t)(P.Zv * KMAX * (int)sizeof(Key)));
#pragma unroll
    for (int i = 0; i < S2_PREFETCH; ++i) {
        const uint32_t o = (uint32_t)((wave + S2_WAVES * i) * KMAX + lane) * (uint32_t)sizeof(Key);
        if constexpr (sizeof(Key) == 4) {
            L.pre_lo[i] = buf_u32(sv, o);
            L.pre_hi[i] = buf_u32(sv, o + WAVE * 4u);
        } else {
            L.pre_lo[i] = buf_u64(sv, o);
            L.pre_hi[i] = buf_u64(sv, o + WAVE * 8u);
        }
    }
    // wave 0: the listed tokens' list (used only when the row has lists)
    const auto lv = buf_view(F.listed ? F.listed + (int64_t)row * KMAX : nullptr,
                             (F.listed && wave == 0) ? (uint32_t)(KMAX * 8) : 0u);
    L.listed = WL64{buf_u64(lv, (uint32_t)lane * 8u), buf_u64(lv, (uint32_t)(lane + WAVE) * 8u)};
}

// The row's 128 best as a wave-0 register list; one workgroup barrier.
template <int DT>
__device__ __forceinline__ WL64 row_merge(const Stage2Params& F, const RowParams& rp, int row, S2Shared& sh,
                                          const RowLoads<DT>& L) {
    using Key = typename S1Traits<DT>::Key;
    const Stage1Params& P = F.s1;
    const int lane = lane_id();
    const int wave = threadIdx.x / WAVE;
    const bool has_listed = rp.valid && rp.n_prior + rp.n_bias + draft_hist_len(P, rp.flags, row) > 0;
    const Key* sc = (const Key*)P.scratch + (int64_t)row * P.Zv * KMAX;
    const auto& pre_lo = L.pre_lo;
    const auto& pre_hi = L.pre_hi;
    const WL64 listed = L.listed;

    // fold this wave's tiles: four at a time as a tree
    auto tl = [&](int i) -> WL64 {
        const int t = wave + S2_WAVES * i;
        return WL64{merge_key<DT>(pre_lo[i], t), merge_key<DT>(pre_hi[i], t)};
    };
    const int mine_n = wave < P.Zv ? (P.Zv - wave + S2_WAVES - 1) / S2_WAVES : 0;
    WL64 mine{0ull, 0ull};
    if (mine_n >= 1) mine = tl(0);
    if (DT == SS_BF16 && mine_n == 2) {
        // two bf16 tiles merge on their 32-bit keys: bit 15 of the low half
        // is always set (local < 2^15) and is cleared on the second tile's
        // keys, so that equal values rank the first tile (lower ids) first;
        // a valid key's high half is never 0, so no key becomes "no token"
        const WList<uint32_t> a{(uint32_t)pre_lo[0], (uint32_t)pre_hi[0]};
        const WList<uint32_t> c{(uint32_t)pre_lo[1] & ~0x8000u, (uint32_t)pre_hi[1] & ~0x8000u};
        const WList<uint32_t> m = wave_merge(a, c);
        auto widen = [&](uint32_t k) -> uint64_t {   // the tile comes back from bit 15
            return k ? merge_key<DT>((typename S1Traits<DT>::Key)(k | 0x8000u), (k & 0x8000u) ? wave : wave + S2_WAVES)
                     : 0ull;
        };
        mine = WL64{widen(m.lo), widen(m.hi)};
    } else if (mine_n >= 2) {
        WL64 a = tl(1);
        if (mine_n >= 3) {
            WL64 c = tl(2);
            if (mine_n >= 4) c = wave_merge(c, tl(3));
            mine = wave_merge(mine, c);   // pairs (0,1) and (2,3) are independent
        }
        mine = wave_merge(mine, a);
    }
    for (int t = wave + S2_WAVES * S2_PREFETCH; t < P.Zv; t += S2_WAVES)   // long vocabularies
        mine = wave_merge(mine, WL64{merge_key<DT>(sc[(int64_t)t * KMAX + lane], t),
                                     merge_key<DT>(sc[(int64_t)t * KMAX + lane + WAVE], t)});
    if (wave == 0 && has_listed) mine = wave_merge(mine, listed);
    sh.wl[wave][0][lane] = mine.lo;
    sh.wl[wave][1][lane] = mine.hi;
    __syncthreads();

    // cross-wave tree: wave 0 takes wave 1's list while wave 1 merges
    // waves 2 and 3; then wave 0 merges the two
    const int nw = min(S2_WAVES, P.Zv);   // block-uniform
    auto wl = [&](int w) -> WL64 { return WL64{sh.wl[w][0][lane], sh.wl[w][1][lane]}; };
    WL64 res = mine;
    if (wave == 0 && nw >= 2) res = wave_merge(res, wl(1));
    if (nw >= 3) {
        if (wave == 1) {
            WL64 z = wl(2);
            if (nw >= 4) z = wave_merge(z, wl(3));
            sh.wl[2][0][lane] = z.lo;
            sh.wl[2][1][lane] = z.hi;
        }
        __syncthreads();
        if (wave == 0) res = wave_merge(res, wl(2));
    }
    return res;
}

// ---------------------------------------------------------------------------
// Verification rules (SonicSampler section 3.1 "Speculative verification";
// the decoding notes' "Rejection Sampler"), applied in two places: Stage 2
// itself (each target row decides its own position; the request's last row
// to arrive finds where it stops from the positions' accept and all-masked
// bits) and verify_kernel (one workgroup per request, from the rows'
// records, for batches above the workspace's word area; emit_request).
// ---------------------------------------------------------------------------

// Request b's draft count: gamma, or n_b = cu[b] - cu[b-1] with per-request
// counts (a count outside [0, gamma] makes the request invalid).  Uniform.
struct DraftCount {
    int n;
    bool ok;
};
__device__ __forceinline__ DraftCount draft_count(const Stage2Params& F, int b) {
    if (!F.cu_num_draft) return DraftCount{F.gamma, true};
    const int hi = F.cu_num_draft[b];
    const int lo = b > 0 ? F.cu_num_draft[b - 1] : 0;
    const bool ok = hi - lo >= 0 && hi - lo <= F.gamma;
    return DraftCount{ok ? hi - lo : 0, ok};
}

// The request's 64-bit word while its rows decide in Stage 2: accept bits
// 0..gamma, all-masked bits 17..17+gamma, the arrival count from bit 48.
constexpr int VF_MASKED_SHIFT = SS_GAMMA_MAX + 1;
constexpr int VF_COUNT_SHIFT = 48;
static_assert(VF_MASKED_SHIFT + SS_GAMMA_MAX + 1 <= VF_COUNT_SHIFT, "decision word layout");

// Position j of request b (whole wave; ranks lane and lane + 64): the row's
// status, greedy flag, kept count n, Gumbel-max token and best id, the
// draft d, the candidates (id -1 past the row's K), their p (0 past n) and
// v, and q gathered at the candidates and at d.  Bonus position (j = n_b):
// the row's token.  Greedy: accept iff d is the best id, else emit the best
// id.  Otherwise accept iff q(d) > 0 and u q(d) <= p(d), u from Philox
// counter {0, b, (1 << 24) | j}; on rejection the Gumbel-max of ln(rho) +
// g over rho = max(0, p - q) > 0 with g from counter {id, b, (2 << 24) | j},
// or of v + g when rho vanishes on every kept candidate.
struct PosDecision {
    int accept;
    int token;
};
// The random numbers position j of request b may use: the acceptance
// uniform and the residual draw's Gumbel noise of the lane's two ranks.
// They depend only on (b, j) and the candidate ids, so a caller can work
// them out before it knows p and q.
struct PosNoise {
    float u;
    float g_lo, g_hi;
};
__device__ __forceinline__ PosNoise position_noise(const ss_rng rg, int b, int j, int id_lo, int id_hi) {
    const uint32_t c2 = (2u << 24) | (uint32_t)j;
    PosNoise z;
    z.u = unit_open(philox_w0(rg.seed, rg.offset, 0u, (uint32_t)b, (1u << 24) | (uint32_t)j));
    z.g_lo = gumbel_noise(rg.seed, rg.offset, (uint32_t)id_lo, (uint32_t)b, c2);
    z.g_hi = gumbel_noise(rg.seed, rg.offset, (uint32_t)id_hi, (uint32_t)b, c2);
    return z;
}
__device__ __forceinline__ PosDecision decide_position(int b, int j, int n_b, int status,
                                                       int greedy, int n, int rtoken, int best, int d, int id_lo_r,
                                                       int id_hi_r, float p_lo_r, float p_hi_r, float v_lo,
                                                       float v_hi, float q_lo_r, float q_hi_r, float q_d_r, int V,
                                                       const PosNoise& nz) {
    const int lane = lane_id();
    int accept = 0, token = -1;
    const bool live = status == SS_ROW_OK || status == SS_ROW_TOPK_CLAMPED;
    if (live && j == n_b) {   // bonus token
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
        accept = qd > 0.0f && nz.u * qd <= pd;
        if (!accept) {
            // draw from norm(max(0, p - q)) by Gumbel-max on ln(rho)
            const float g_lo = id_lo >= 0 ? nz.g_lo : 0.0f;
            const float g_hi = id_hi >= 0 ? nz.g_hi : 0.0f;
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
    return PosDecision{accept, token};
}

// Request b's output from its positions' decisions (one lane): the accepted
// drafts in order, then the first rejection's draw or the bonus token; -1
// after; a request whose first row is invalid (or whose count is) emits
// nothing, and one whose emitted path meets an all-masked row stops there.
__device__ __forceinline__ void emit_request(const Stage2Params& F, int b, const DraftCount& dc, const int* acc,
                                             const int* tok, const int* st) {
    const int G = F.gamma;
    int32_t* out = F.v_tokens + (int64_t)b * (G + 1);
    int emitted = 0;
    int status;
    if (!dc.ok || st[0] == SS_ROW_INVALID) {
        status = SS_ROW_INVALID;
    } else {
        status = st[0] == SS_ROW_TOPK_CLAMPED ? SS_ROW_TOPK_CLAMPED : SS_ROW_OK;
        for (int j = 0; j <= dc.n; ++j) {
            if (st[j] == SS_ROW_ALL_MASKED) {
                status = SS_ROW_ALL_MASKED;
                break;
            }
            if (j < dc.n && acc[j]) {
                out[emitted++] = F.draft_ids[(int64_t)b * G + j];
                continue;
            }
            out[emitted++] = tok[j];   // first rejection's draw, or the bonus
            break;
        }
    }
    for (int j = emitted; j <= G; ++j) out[j] = -1;
    F.v_n_emit[b] = emitted;
    if (F.v_status) F.v_status[b] = status;
}

// What verification in Stage 2 can request before the merge: the request's
// draft count and position j's draft (any value past the count: not used).
// They depend only on (request, position), so they are requested at the
// start of the workgroup and arrive during the merge; q at the draft waits
// for the epilogue, with q at the candidates, so no wave waits for the
// draft early.
struct VerifyPre {
    DraftCount dc;
    int d;
};
__device__ __forceinline__ VerifyPre verify_pre(const Stage2Params& F, int row, int b) {
    const int G = F.gamma;
    const int j = row - b * F.s1.rows_per_req;
    VerifyPre vp;
    vp.d = j < G ? F.draft_ids[(int64_t)b * G + j] : -1;
    vp.dc = draft_count(F, b);
    return vp;
}

// Epilogue on wave 0 (ranks k = lane and lane + 64).  Writes the mode's
// outputs for the row.  Uses no barrier.
template <int DT, int MODE>
__device__ __forceinline__ void row_epilogue(const Stage2Params& F, const RowParams& rp, int row, int b, const WL64& best,
                             const ss_rng rg, S2Shared& sh, const VerifyPre& vp) {
    const Stage1Params& P = F.s1;
    const int lane = lane_id();
    const uint64_t k_lo = best.lo, k_hi = best.hi;
    const int id_lo = key_id(k_lo), id_hi = key_id(k_hi);
    const float z_lo = key_z(k_lo), z_hi = key_z(k_hi);
    const uint64_t k0 = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)k_lo) |
                        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(k_lo >> 32)) << 32);
    const int id0 = key_id(k0);
    const float z0 = key_z(k0);
    const float NINF = bitsf(F32_NINF_BITS);
    // verification decided in this launch: the draft probabilities at the
    // candidates and at the draft (requested with the lists) are requested
    // first, so that they arrive while the epilogue runs
    const int vj = row - b * P.rows_per_req;
    const DraftCount dc = vp.dc;
    const int vd = vj < dc.n ? vp.d : -1;
    float q_lo_r = 0.0f, q_hi_r = 0.0f, q_d_r = 0.0f;
    if constexpr (MODE == MODE_VERIFY) {
        if (F.arrive) {
            const float* q = F.draft_probs + ((int64_t)b * F.gamma + (vj < F.gamma ? vj : F.gamma - 1)) * P.V;
            auto in_v = [&](int id) { return (unsigned)id < (unsigned)P.V; };
            q_lo_r = q[in_v(id_lo) ? id_lo : 0];
            q_hi_r = q[in_v(id_hi) ? id_hi : 0];
            q_d_r = q[in_v(vd) ? vd : 0];
        }
    }

    if constexpr (MODE == MODE_TOPK) {
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
    PosNoise pz{0.0f, 0.0f, 0.0f};   // verification: the position's noise (stochastic rows)
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
        // ranks past K keep v = -inf, e = 0 (selected, so that the code
        // below has no branch)
        const bool in_lo = lane < K, in_hi = lane + 64 < K;
        {
            const float vl = vscale(z_lo), vh = vscale(z_hi);
            // v - m <= 0 (m is the best value; a live row's m is finite)
            const float el = exp_fixed_nonpos(vl - m), eh = exp_fixed_nonpos(vh - m);
            v_lo = in_lo ? vl : NINF;
            v_hi = in_hi ? vh : NINF;
            e_lo = in_lo ? el : 0.0f;
            e_hi = in_hi ? eh : 0.0f;
        }
        uint32_t c1, c2;
        if constexpr (MODE == MODE_VERIFY) {
            c1 = (uint32_t)b;
            c2 = (uint32_t)(row - b * P.rows_per_req);
        } else {
            c1 = (uint32_t)row;
            c2 = 0u;
        }
        // running sums E_k = e_0 + ... + e_{k-1}, left to right: the e's go
        // to LDS and every lane runs the same dependent chain on broadcast
        // reads (ranks past K hold e = 0, which leaves E unchanged); lane k
        // keeps E_k and E_{k+64}.  The Gumbel noise of both candidates is
        // worked out in the same straight-line block, so that its dependent
        // chains and the sum's fill each other's latency.
        float* es = (float*)&sh.wl[0][0][0];   // waves 1-3 are done with sh
        es[lane] = e_lo;
        es[lane + WAVE] = e_hi;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        float4 eq[KMAX / 4];
#pragma unroll
        for (int i = 0; i < KMAX / 4; ++i) eq[i] = *(const float4*)&es[4 * i];
        const float gl = gumbel_noise(rg.seed, rg.offset, (uint32_t)id_lo, c1, c2);
        const float gh = gumbel_noise(rg.seed, rg.offset, (uint32_t)id_hi, c1, c2);
        if constexpr (MODE == MODE_VERIFY)   // the decision's noise, ahead of p and q
            if (F.arrive) pz = position_noise(rg, b, vj, id_lo, id_hi);
        float E = 0.0f, E_lo = 0.0f, E_hi = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const float4 q = eq[k / 4];
            const float ek = (k & 3) == 0 ? q.x : (k & 3) == 1 ? q.y : (k & 3) == 2 ? q.z : q.w;
            const bool mine = __builtin_amdgcn_inverse_ballot_w64(1ull << (k & 63));   // lane == k mod 64
            if (k < WAVE) E_lo = mine ? E : E_lo;
            else E_hi = mine ? E : E_hi;
            E = E + ek;
        }
        const float g_lo = in_lo ? gl : 0.0f, g_hi = in_hi ? gh : 0.0f;
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
        float s_lo = 0.0f, s_hi = 0.0f;
        const bool c_lo = lane < n, c_hi = lane + 64 < n;
        if (c_lo) s_lo = v_lo + g_lo;
        if (c_hi) s_hi = v_hi + g_hi;
        // best of the lane's two, then across the wave
        float s = s_lo;
        int id = c_lo ? id_lo : -1;
        if (c_hi && (id < 0 || s_hi > s || (s_hi == s && id_hi < id))) {
            s = s_hi;
            id = id_hi;
        }
        token = wave_argmax(s, id, id >= 0);
    }

    if constexpr (MODE == MODE_SAMPLE) {
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
    } else if (F.arrive) {   // MODE_VERIFY, decided here
        const int n_r = live ? n : 0;
        const int idl = (status != SS_ROW_INVALID && lane < K) ? id_lo : -1;
        const int idh = (status != SS_ROW_INVALID && lane + 64 < K) ? id_hi : -1;
        const float pl = (live && !rp.greedy && lane < n) ? e_lo / En : 0.0f;
        const float ph = (live && !rp.greedy && lane + 64 < n) ? e_hi / En : 0.0f;
        const int best_id = __builtin_amdgcn_readfirstlane(idl);
        const PosDecision pd = decide_position(b, vj, dc.n, status, rp.greedy, n_r, token, best_id, vd, idl, idh,
                                               pl, ph, v_lo, v_hi, q_lo_r, q_hi_r, q_d_r, P.V, pz);
        // Position j's output slot holds the draft if it was accepted, else
        // this row's draw: what the request emits there whenever every
        // earlier draft is accepted.  The row writes it (device-coherent,
        // completed before the arrival), then adds its arrival, its accept
        // bit (bit j) and its all-masked bit (bit 17 + j) to the request's
        // 64-bit word; the last arrival has every position's bits from the
        // add's return value, finds where the request stops, and writes -1
        // past it (also device-coherent, so that it lands after the rows'
        // writes), the count and the status.  (The step's Stage-1 launch
        // zeroed the word.)
        if (lane == 0) {
            const int G = F.gamma;
            int32_t* out = F.v_tokens + (int64_t)b * (G + 1);
            const bool acc = vj < dc.n && pd.accept;
            store_coherent(out + vj, acc ? vd : pd.token);
            wait_memory();
            const uint64_t mine = (1ull << VF_COUNT_SHIFT) | ((uint64_t)acc << vj) |
                                  ((uint64_t)(status == SS_ROW_ALL_MASKED) << (VF_MASKED_SHIFT + vj));
            uint64_t* word = (uint64_t*)F.arrive + b;
            const uint64_t old = __hip_atomic_fetch_add(word, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int arrivals = (dc.ok ? dc.n : G) + 1;
            if ((int)(old >> VF_COUNT_SHIFT) + 1 == arrivals) {
                const uint64_t all = old + mine;
                int emitted = 0, st = SS_ROW_INVALID;
                if (dc.ok && status != SS_ROW_INVALID) {   // validity is per request
                    st = rp.clamped ? SS_ROW_TOPK_CLAMPED : SS_ROW_OK;
                    for (int j = 0; j <= dc.n; ++j) {
                        if ((all >> (VF_MASKED_SHIFT + j)) & 1ull) {
                            st = SS_ROW_ALL_MASKED;   // nothing emitted here (the row wrote -1)
                            break;
                        }
                        emitted = j + 1;
                        if (j == dc.n || !((all >> j) & 1ull)) break;
                    }
                }
                for (int j = emitted; j <= G; ++j) store_coherent(out + j, -1);
                F.v_n_emit[b] = emitted;
                if (F.v_status) F.v_status[b] = st;
            }
        }
    } else {   // MODE_VERIFY, records for verify_kernel
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

template <int DT, int MODE>
__global__ __launch_bounds__(S2_THREADS) void stage2_kernel(Stage2Params F) {
    __shared__ S2Shared sh;
    const int row = blockIdx.x;
    if (!row_used(F.s1, row)) return;
    const int b = __builtin_amdgcn_readfirstlane(div_uniform(row, F.s1.rows_per_req));
    RowLoads<DT> L;
    row_loads<DT>(F, row, L);   // the Stage-1 lists first
    VerifyPre vp{DraftCount{0, true}, -1};
    if constexpr (MODE == MODE_VERIFY)
        if (F.arrive) vp = verify_pre(F, row, b);
    ss_rng rg{0ull, 0ull};
    if (F.rng) rg = *F.rng;
    const RowParams rp = row_params(F.s1, b, &L.bias_head, L.rq);
    const WL64 best = row_merge<DT>(F, rp, row, sh, L);
    if (threadIdx.x >= WAVE) return;
    row_epilogue<DT, MODE>(F, rp, row, b, best, rg, sh, vp);
}

}  // namespace ssd
