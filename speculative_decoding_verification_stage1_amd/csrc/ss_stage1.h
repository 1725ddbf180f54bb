// Stage 1 of the two-stage tile-aware top-k (SonicSampler section 3.2 and
// Fig. 1, stage 1): one workgroup per (row, vocabulary tile of BN tokens).
// The workgroup streams the tile once, applies the per-token part of the
// logits processing (grammar mask; tokens named by a penalty or bias list
// are left out here and ranked in Stage 2), and writes the tile's 128 best
// tokens, sorted best first, as packed order keys to the workspace - the
// only data that crosses to Stage 2.
//
// Packed key (larger = better, unique per token of the tile):
//   bf16 rows: uint32 (ord16(value) << 16) | (0xFFFF - local)
//   fp32 rows: uint64 (ord32(value) << 32) | (0xFFFFFFFF - local)
// where `local` is the token's index inside the tile.  Key 0 means "no
// token" (tail of a short tile).  Ties in value therefore rank the lower
// token id first, the order used throughout.
//
// Selection is exact.  Fast path: raw bit patterns read as signed integers
// order like the floats they hold whenever the threshold below is positive,
// so no per-element key transform is needed.  Grammar-masked elements and
// those past the end of V take the smallest pattern.  Each lane holds 16
// chunks of 16 bytes and takes the maximum of every chunk and of its whole
// slice; each wave finds the k-th largest of its 64 lane maxima, k = 32 +
// ceil(L/4) for L listed tokens in the tile, and the smallest of the four is
// a threshold tau with at least 128 + L tokens at or above it - so the 128
// best unlisted tokens are all at or above tau.  Chunks whose maximum
// reaches tau (typically a few dozen per wave) are copied from registers to
// the wave's LDS area; each lane then takes one such chunk, and its elements
// >= tau that are not listed become keys, one per lane per round.  Each
// wave sorts its keys in registers, and a two-level merge tree gives the
// tile's 128.  Tiles where the test does not apply (tau <= 0, a positive
// NaN, more listed tokens or survivors than the LDS areas hold) take the
// general path: exact keys for every element and a bisection for the 128th
// key.
#pragma once

#include "ss_device.h"
#include "ss_wavesort.h"

namespace ssd {

typedef short s16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ s16x2 bits_s16x2(uint32_t u) { return __builtin_bit_cast(s16x2, u); }
__device__ __forceinline__ uint32_t s16x2_bits(s16x2 v) { return __builtin_bit_cast(uint32_t, v); }

constexpr int S1_THREADS = 256;
constexpr int S1_WAVES = S1_THREADS / WAVE;
constexpr int S1_CPT = 16;            // 16-byte chunks per thread
constexpr int S1_CCAP = 128;          // flagged chunks held per wave (fast path)
constexpr int S1_KCAP = 256;          // survivors held per wave (fast path)
constexpr int S1_LIST_CAP = 528;      // >= 255 prior + 255 bias entries + SS_GAMMA_MAX drafts
constexpr int S1_NL_FAST = 128;       // listed tokens per tile the fast path absorbs

template <int DT> struct S1Traits;
template <> struct S1Traits<SS_BF16> {
    using Key = uint32_t;
    static constexpr int EPC = 8;                            // elements per chunk
    static constexpr int BN = EPC * S1_CPT * S1_THREADS;     // tile width 32768
    static constexpr int VAL_BITS = 16;                      // fast-path value range (int16)
};
template <> struct S1Traits<SS_F32> {
    using Key = uint64_t;
    static constexpr int EPC = 4;
    static constexpr int BN = EPC * S1_CPT * S1_THREADS;     // 16384
    static constexpr int VAL_BITS = 32;
};

struct Stage1Params {
    const void* logits;
    int64_t ld;
    int V;
    int rows;
    int Zv;
    int rows_per_req;
    const ss_req* req;   // may be null: no processing
    ss_aux aux;
    void* scratch;       // keys [rows][Zv][128]
    int32_t* out_ids;    // optional [rows][Zv][128]
    uint64_t* listed;    // [rows][128] listed tokens' merge keys (sampling / verification)
    int listed_rows;     // rows 0 .. listed_rows-1 need them (one wave per row)
    int aligned16;       // rows start on 16-byte boundaries
    ss_rng* rng;         // sampling / verification: the caller's generator state
    ss_rng* rng_snap;    // ... copied here for Stage 2 (workgroup 0)
    uint64_t rng_advance;   // ... after which rng->offset += rng_advance
    const int32_t* cu_num_draft;   // verification with per-request draft counts (or null)
    const int32_t* draft_ids;      // verification: [requests, rows_per_req - 1] drafts (or null)
    uint64_t* clear_words;         // verification: decision words zeroed by workgroup 0 (or null)
    int n_clear;
};

// Number of earlier drafts in row `row`'s penalty history: its position j
// when the request asks for the draft history and applies penalties, else
// 0.  Uniform per row.
__device__ __forceinline__ int draft_hist_len(const Stage1Params& P, uint32_t flags, int row) {
    if (!P.draft_ids || !(flags & SS_DRAFT_HIST) || !(flags & (SS_REP | SS_FREQPRES))) return 0;
    const int b = div_uniform(row, P.rows_per_req);
    return row - b * P.rows_per_req;
}

// Whether row `row` takes part: always, except in verification with
// per-request draft counts, where request b's rows past its bonus position
// n_b are not used (a count outside [0, rows_per_req - 1] leaves every row
// in: the request is reported invalid).  Uniform per workgroup.
__device__ __forceinline__ bool row_used(const Stage1Params& P, int row) {
    if (!P.cu_num_draft) return true;
    const int b = div_uniform(row, P.rows_per_req);
    const int j = row - b * P.rows_per_req;
    const int n = P.cu_num_draft[b] - (b > 0 ? P.cu_num_draft[b - 1] : 0);
    return n < 0 || n >= P.rows_per_req || j <= n;
}

// Largest t such that at least k lanes of the wave hold m >= t (signed).
// Bisection on the biased value, one ballot per bit.
template <int BITS>
__device__ __forceinline__ int wave_kth_largest(int m, int k) {
    if (BITS == 16) {
        const uint32_t u = (uint32_t)(m + 32768);
        uint32_t res = 0;
#pragma unroll
        for (int bit = 15; bit >= 0; --bit) {
            const uint32_t cand = res | (1u << bit);
            if (__popcll(__ballot(u >= cand)) >= k) res = cand;
        }
        return (int)res - 32768;
    } else {
        const uint32_t u = (uint32_t)m ^ 0x80000000u;
        uint32_t res = 0;
#pragma unroll
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = res | (1u << bit);
            if (__popcll(__ballot(u >= cand)) >= k) res = cand;
        }
        return (int)(res ^ 0x80000000u);
    }
}

// Block-wide exclusive scan of one int per thread; returns the prefix and
// writes the total to *total (all threads).  Uses `tmp` [S1_WAVES] in LDS.
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
    const int w = threadIdx.x / WAVE;
    const int incl = wave_incl_scan(v);
    if (lane_id() == WAVE - 1) tmp[w] = incl;
    __syncthreads();
    int before = 0, sum = 0;
#pragma unroll
    for (int i = 0; i < S1_WAVES; ++i) {
        const int t = tmp[i];
        if (i < w) before += t;
        sum += t;
    }
    __syncthreads();
    *total = sum;
    return before + incl - v;
}

// Exact key of one element of a bf16 tile.
__device__ __forceinline__ uint32_t key_bf16(uint32_t raw16, int local, bool present, bool allowed) {
    if (!present) return 0u;
    const uint32_t k16 = allowed ? ord16_canon(raw16) : K16_NINF;
    return (k16 << 16) | (0xFFFFu - (uint32_t)local);
}
__device__ __forceinline__ uint64_t key_f32(uint32_t raw, int local, bool present, bool allowed) {
    if (!present) return 0ull;
    const uint32_t k32 = allowed ? ord32(canon(bitsf(raw))) : ord32(bitsf(F32_NINF_BITS));
    return ((uint64_t)k32 << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)local);
}

template <int DT>
struct S1Shared {
    using Key = typename S1Traits<DT>::Key;
    uint4 chunks[S1_WAVES][S1_CCAP + WAVE];   // flagged chunks, per wave (fast path)
    int cid[S1_WAVES][S1_CCAP + WAVE];        // their chunk index in the tile
    Key keys[S1_WAVES][S1_KCAP];       // survivors per wave (fast path); general path: flat
    Key wl[S1_WAVES][KMAX];            // per-wave sorted lists
    Key surv[KMAX];                    // result: the tile's 128 best, sorted
    uint4 gtab[256];                   // bf16 grammar: dword masks of a chunk by its allowed byte
    uint32_t gmw[S1Traits<DT>::BN / 32];   // the tile's grammar bitmask
    int listed[S1_LIST_CAP];           // tile-local index of each listed token
    int2 lcb[S1_LIST_CAP];             // its chunk, and its bit in a chunk's survivor mask
    int nl;
    int tau[S1_WAVES];
    int special[S1_WAVES];
    int ovf;
    int scan[S1_WAVES];
    int red[2][S1_WAVES];
};

// Orders one wave's LDS writes before its later LDS reads of other lanes'
// entries (a wave's LDS operations complete in issue order).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// The best 128 of n keys held in LDS by one wave, sorted, as a wave list.
template <typename Key>
__device__ __forceinline__ WList<Key> wave_top128(const Key* keys, int n) {
    const int lane = lane_id();
    WList<Key> mine{0, 0};
    if (n <= WAVE) {
        Key k = lane < n ? keys[lane] : (Key)0;
        wave_sort64(k);
        mine.lo = k;
        return mine;
    }
    for (int c0 = 0; c0 < n; c0 += KMAX) {
        const int i0 = c0 + lane, i1 = i0 + WAVE;
        WList<Key> l{i0 < n ? keys[i0] : (Key)0, i1 < n ? keys[i1] : (Key)0};
        l = wave_sort128(l);
        mine = c0 == 0 ? l : wave_merge(mine, l);
    }
    return mine;
}

// Bit of element e of a chunk in the survivor mask of that chunk.  bf16:
// element 2k (low half of dword k) is bit 15 - k, element 2k + 1 is bit
// 31 - k (the sign bits of a packed subtraction, see chunk_survivors).
template <int DT>
__device__ __forceinline__ uint32_t chunk_bit(int e) {
    if constexpr (DT == SS_BF16) return 1u << ((15 - (e >> 1)) + 16 * (e & 1));
    else return 1u << e;
}
template <int DT>
__device__ __forceinline__ int chunk_elem(int p) {
    if constexpr (DT == SS_BF16) return 2 * (15 - (p & 15)) + (p >> 4);
    else return p;
}
// Elements of a chunk whose value (raw pattern read as signed) is >= tau.
template <int DT>
__device__ __forceinline__ uint32_t chunk_survivors(const uint4& d, int tau) {
    if constexpr (DT == SS_BF16) {
        const s16x2 t2 = {(short)tau, (short)tau};
        const uint32_t w[4] = {d.x, d.y, d.z, d.w};
        uint32_t below = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k)   // saturating: the sign says x < tau
            below |= (s16x2_bits(__builtin_elementwise_sub_sat(bits_s16x2(w[k]), t2)) & 0x80008000u) >> k;
        return ~below & 0xF000F000u;
    } else {
        return ((int)d.x >= tau ? 1u : 0u) | ((int)d.y >= tau ? 2u : 0u) | ((int)d.z >= tau ? 4u : 0u) |
               ((int)d.w >= tau ? 8u : 0u);
    }
}

// What one tile needs from global memory, all requested before any of it
// is used.
template <int DT>
struct S1In {
    uint32_t raw[S1_CPT * 4];   // dword q: dword (q & 3) of this thread's chunk (q >> 2)
    uint32_t gw[S1_CPT * S1Traits<DT>::EPC / 32];   // the tile's bitmask words tid + 256k
    int l_pid, l_pct, l_bid;    // lead wave: first 64 entries of the request's lists
    int l_did;                  // lead wave: draft `lane` of the request (verification), or -1
    uint32_t rq_flags, rq_lists; // the request's flags and its n_prior | n_bias << 8
};

__device__ __forceinline__ int s1_lead_wave() { return (int)((blockIdx.x >> 3) & (S1_WAVES - 1)); }

#define S1_TILE_GEOMETRY                                                             \
    using T = S1Traits<DT>;                                                          \
    constexpr int EPC = T::EPC;                                                      \
    constexpr int BN = T::BN;                                                        \
    constexpr int CPT = S1_CPT;                                                      \
    constexpr int NQ = CPT * 4;                                                      \
    constexpr uint32_t PAD = DT == SS_BF16 ? 0x80008000u : 0x80000000u;              \
    const int tid = threadIdx.x;                                                     \
    const int wave = tid / WAVE;                                                     \
    /* the wave that reads the lists, merges last and holds the result: it   \
       rotates with the workgroup index, so that the workgroups sharing a    \
       compute unit put this extra work on different SIMDs */                \
    const int lead = s1_lead_wave();                                                 \
    const int lane = lane_id();                                                      \
    const int base = tile * BN;                                                      \
    const int nvalid = min(BN, P.V - base);                                          \
    const int b = __builtin_amdgcn_readfirstlane(div_uniform(row, P.rows_per_req));  \
    const bool full = (nvalid == BN);                                                \
    const bool vec = full && P.aligned16;                                            \
    const char* rowp = (const char*)P.logits + ((int64_t)row * P.ld + base) * (DT == SS_BF16 ? 2 : 4); \
    (void)wave; (void)lead; (void)lane; (void)b; (void)vec; (void)NQ; (void)PAD;

// Dword q of this thread's slice (chunk q >> 2, dword q & 3); elements past
// the end of V read as the smallest signed pattern.
template <int DT>
__device__ __forceinline__ uint32_t tile_dword(const char* rowp, bool vec, int nvalid, int q) {
    constexpr int EPC = S1Traits<DT>::EPC;
    const int c = (q >> 2) * S1_THREADS + (int)threadIdx.x;
    if (vec) return gmem((const uint32_t*)rowp)[c * 4 + (q & 3)];
    if (DT == SS_BF16) {
        const auto p16 = gmem((const uint16_t*)rowp);
        const int e0 = c * EPC + 2 * (q & 3);
        const uint32_t lo = e0 < nvalid ? p16[e0] : 0x8000u;
        const uint32_t hi = e0 + 1 < nvalid ? p16[e0 + 1] : 0x8000u;
        return lo | (hi << 16);
    } else {
        const int e = c * EPC + (q & 3);
        return e < nvalid ? gmem((const uint32_t*)rowp)[e] : 0x80000000u;
    }
}

// Requests tile `tile` of row `row`: chunk j of thread t is tile chunk
// j*256 + t (each wave instruction reads 1 KiB of consecutive bytes).
template <int DT>
__device__ __forceinline__ void tile_fetch(const Stage1Params& P, int row, int tile, S1In<DT>& in) {
    S1_TILE_GEOMETRY
    // the lead wave: the first 64 entries of the request's lists
    in.l_pid = -1;
    in.l_pct = 0;
    in.l_bid = -1;
    if (wave == lead) {
        if (P.aux.prior_ids && P.aux.prior_cnt && lane < P.aux.prior_stride) {
            const int64_t o = (int64_t)b * P.aux.prior_stride + lane;
            in.l_pid = gmem(P.aux.prior_ids)[o];
            in.l_pct = gmem(P.aux.prior_cnt)[o];
        }
        if (P.aux.bias_ids && lane < P.aux.bias_stride)
            in.l_bid = gmem(P.aux.bias_ids)[(int64_t)b * P.aux.bias_stride + lane];
    }
    in.l_did = -1;
    if (wave == lead && P.draft_ids) {   // drafts before this row's position (read if the flag asks)
        const int j = row - b * P.rows_per_req;
        if (lane < j) in.l_did = gmem(P.draft_ids)[(int64_t)b * (P.rows_per_req - 1) + lane];
    }
    // the tile's grammar bitmask, coalesced: word base/32 + tid + 256k
    // (requested before the logits, so that it can be used while they arrive)
    if (P.aux.bitmask) {
        constexpr int GW = CPT * EPC / 32;
        const int words = (P.V + 31) / 32;
        const auto gm = gmem(P.aux.bitmask + (int64_t)row * P.aux.bitmask_stride) + base / 32 + tid;
#pragma unroll
        for (int k = 0; k < GW; ++k)
            in.gw[k] = (full || base / 32 + tid + k * S1_THREADS < words) ? __builtin_nontemporal_load(gm + k * S1_THREADS) : 0u;
    }
    // the logits, as one buffer view over the tile's whole 16-byte chunks:
    // the same 16 loads for every tile, with nothing between them, so that
    // each chunk can be used as soon as it has arrived.  Chunks past V (and
    // every chunk of a row that does not start on a 16-byte boundary) read
    // as zero without touching memory; tile_patch sets them.  The whole
    // offset is in the lane's offset, which the range check covers.
    const int nbytes = P.aligned16 ? (nvalid / EPC) * 16 : 0;
    const __amdgpu_buffer_rsrc_t rs = buf_view(rowp, (uint32_t)nbytes);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const vu32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, (tid + j * S1_THREADS) * 16, 0, LD_STREAM);
        __builtin_amdgcn_sched_barrier(0);   // keep the issue order: chunk j is used j-th
        in.raw[4 * j + 0] = v.x;
        in.raw[4 * j + 1] = v.y;
        in.raw[4 * j + 2] = v.z;
        in.raw[4 * j + 3] = v.w;
    }
    __builtin_amdgcn_sched_barrier(0);
    // the request's flags and list lengths last, through the scalar cache:
    // nothing above waits for them
    in.rq_flags = 0;
    in.rq_lists = 0;
    if (P.req) {
        const auto rq = (const uint32_t*)(P.req + b);
        in.rq_flags = rq[0];
        in.rq_lists = rq[2] >> 16;   // n_prior, n_bias follow the 16-bit top_k
    }
}

// Tiles that are not whole 16-byte chunks of an aligned row: chunks not
// wholly inside V become PAD, and the one that straddles the end is
// completed by its owner thread from the elements inside V (rows that do
// not start on a 16-byte boundary are all PAD: the exact general path reads
// their elements itself).  Waits for the tile's loads, so full tiles skip it.
template <int DT>
__device__ __forceinline__ void tile_patch(const Stage1Params& P, int row, int tile, S1In<DT>& in) {
    S1_TILE_GEOMETRY
    if (vec) return;
    const int cp = P.aligned16 ? nvalid / EPC : 0;   // first chunk not wholly inside V
#pragma unroll
    for (int j = 0; j < CPT; ++j)
        if (j * S1_THREADS + tid >= cp) {
#pragma unroll
            for (int k = 0; k < 4; ++k) in.raw[4 * j + k] = PAD;
        }
    if (!P.aligned16) return;
    const int rem = nvalid - cp * EPC;   // its elements inside V
    if (rem == 0 || (cp & (S1_THREADS - 1)) != tid) return;
    uint32_t pv[4] = {PAD, PAD, PAD, PAD};
#pragma unroll
    for (int k = 0; k < EPC; ++k) {
        if (k < rem) {
            if constexpr (DT == SS_BF16) {
                const uint32_t h = gmem((const uint16_t*)rowp)[cp * EPC + k];
                const int sft = 16 * (k & 1);
                pv[k >> 1] = (pv[k >> 1] & ~(0xFFFFu << sft)) | (h << sft);
            } else {
                pv[k] = gmem((const uint32_t*)rowp)[cp * EPC + k];
            }
        }
    }
    const int jp = cp / S1_THREADS;
#pragma unroll
    for (int j = 0; j < CPT; ++j)
        if (j == jp) {
#pragma unroll
            for (int k = 0; k < 4; ++k) in.raw[4 * j + k] = pv[k];
        }
}

// The 128 best tokens of tile `tile` of row `row` (whose data `in` holds),
// sorted best first (key 0 = no token): left in sh.surv[0..128) behind a
// final barrier, or, with `to_regs`, handed to the lead wave's registers
// with no final barrier (the other waves return early).  `next()` is called
// as soon as the registers of `in` are no longer needed (the candidate
// chunks are in LDS by then).
template <int DT, typename Next>
__device__ __forceinline__ void tile_process(const Stage1Params& P, int row, int tile, S1In<DT>& in,
                                             S1Shared<DT>& sh, Next&& next,
                                             WList<typename S1Traits<DT>::Key>* to_regs = nullptr) {
    S1_TILE_GEOMETRY
    using Key = typename T::Key;
    static_assert(S1_WAVES == 4, "merge tree");
    uint32_t(&raw)[NQ] = in.raw;
    auto load_dword = [&](int q) -> uint32_t { return tile_dword<DT>(rowp, vec, nvalid, q); };

    const uint32_t flags = __builtin_amdgcn_readfirstlane(in.rq_flags);
    const uint32_t lists = __builtin_amdgcn_readfirstlane(in.rq_lists);
    // a list longer than its stride makes the row invalid (reported by
    // Stage 2); the tiles then use no list at all
    const int n_prior = (int)(lists & 0xFFu) <= P.aux.prior_stride ? (int)(lists & 0xFFu) : 0;
    const int n_bias = (int)(lists >> 8) <= P.aux.bias_stride ? (int)(lists >> 8) : 0;
    const bool use_grammar = (flags & SS_GRAMMAR) && P.aux.bitmask;
    const bool use_prior = (flags & (SS_REP | SS_FREQPRES)) && P.aux.prior_ids && P.aux.prior_cnt && n_prior > 0;
    const bool use_bias = (flags & SS_BIAS) && P.aux.bias_ids && n_bias > 0;

    // the tile's grammar words go to LDS; each thread then reads the bits
    // of its own chunks
    if (use_grammar) {
#pragma unroll
        for (int k = 0; k < CPT * EPC / 32; ++k) sh.gmw[tid + k * S1_THREADS] = in.gw[k];
        if (DT == SS_BF16) {   // entry tid: bit 2k -> low half of dword k, bit 2k+1 -> high half
            uint32_t mk[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                mk[k] = (((uint32_t)tid >> (2 * k)) & 1u ? 0x0000FFFFu : 0u) |
                        (((uint32_t)tid >> (2 * k + 1)) & 1u ? 0xFFFF0000u : 0u);
            sh.gtab[tid] = make_uint4(mk[0], mk[1], mk[2], mk[3]);
        }
    }
    const int l_pid = in.l_pid, l_pct = in.l_pct, l_bid = in.l_bid;

    // ---- the lead wave: tokens of this tile named by an active list (ranked in
    // Stage 2, left out here) ----
    if (wave == lead) {
        int nl = 0;
        auto record = [&](bool ok, int loc) {
            const uint64_t bal = __ballot(ok);
            if (ok) {
                const int i = nl + lane_prefix(bal);
                sh.listed[i] = loc;
                sh.lcb[i] = make_int2(loc / EPC, (int)chunk_bit<DT>(loc % EPC));
            }
            nl += __popcll(bal);
        };
        // entries 0..63 come from the early request; longer lists load the
        // rest now
        if (use_prior) {
            const int loc = l_pid - base;
            record(lane < n_prior && l_pct >= 1 && l_pid >= 0 && l_pid < P.V && loc >= 0 && loc < nvalid, loc);
            if (n_prior > WAVE) {
                const auto ids = gmem(P.aux.prior_ids + (int64_t)b * P.aux.prior_stride);
                const auto cts = gmem(P.aux.prior_cnt + (int64_t)b * P.aux.prior_stride);
                for (int j0 = WAVE; j0 < n_prior; j0 += WAVE) {
                    const int j = j0 + lane;
                    const int id = j < n_prior ? ids[j] : -1;
                    const int ct = j < n_prior ? cts[j] : 0;
                    const int lc = id - base;
                    record(j < n_prior && ct >= 1 && id >= 0 && id < P.V && lc >= 0 && lc < nvalid, lc);
                }
            }
        }
        if (use_bias) {
            const int loc = l_bid - base;
            record(lane < n_bias && l_bid >= 0 && l_bid < P.V && loc >= 0 && loc < nvalid, loc);
            if (n_bias > WAVE) {
                const auto ids = gmem(P.aux.bias_ids + (int64_t)b * P.aux.bias_stride);
                for (int j0 = WAVE; j0 < n_bias; j0 += WAVE) {
                    const int j = j0 + lane;
                    const int id = j < n_bias ? ids[j] : -1;
                    const int lc = id - base;
                    record(j < n_bias && id >= 0 && id < P.V && lc >= 0 && lc < nvalid, lc);
                }
            }
        }
        // earlier drafts in the penalty history (verification)
        const int nh = draft_hist_len(P, flags, row);
        if (nh > 0) {
            const int loc = in.l_did - base;
            record(lane < nh && in.l_did >= 0 && in.l_did < P.V && loc >= 0 && loc < nvalid, loc);
        }
        if (lane == 0) {
            sh.nl = nl;
            sh.ovf = 0;
        }
    }
    __syncthreads();   // listed tokens, grammar table
    const int nl = sh.nl;
    // grammar rows: the tile's listed tokens are cleared from its grammar
    // words, so the mask leaves them out like any disallowed token and the
    // threshold and survivor steps need not know about them
    const bool fold = use_grammar && nl > 0;   // block-uniform
    if (fold) {
        for (int i = tid; i < nl; i += S1_THREADS) {
            const int loc = sh.listed[i];
            atomicAnd(&sh.gmw[loc >> 5], ~(1u << (loc & 31)));
        }
        __syncthreads();
    }
    const int nl_data = fold ? 0 : nl;   // listed tokens still present in the data

    // ---- grammar mask (masked elements take PAD) and maxima per chunk and
    // per lane (raw patterns read as signed), chunk by chunk in the order
    // the loads were issued, so that each waits only for its own data ----
    uint32_t gbits[CPT];   // bits of chunk j's elements allowed by the grammar (bit e: element e)
    if (use_grammar) {
        const uint8_t* gb = (const uint8_t*)sh.gmw;
#pragma unroll
        for (int j = 0; j < CPT; ++j)
            gbits[j] = DT == SS_BF16 ? gb[j * S1_THREADS + tid]
                                     : (uint32_t)gb[(j * S1_THREADS + tid) >> 1] >> ((tid & 1) * 4);
    }
    uint32_t cmx[CPT];
    auto chunk_max = [&](int j) {
        if constexpr (DT == SS_BF16) {
            const s16x2 a = __builtin_elementwise_max(bits_s16x2(raw[4 * j]), bits_s16x2(raw[4 * j + 1]));
            const s16x2 c = __builtin_elementwise_max(bits_s16x2(raw[4 * j + 2]), bits_s16x2(raw[4 * j + 3]));
            cmx[j] = s16x2_bits(__builtin_elementwise_max(a, c));
        } else {
            cmx[j] = (uint32_t)max(max((int)raw[4 * j], (int)raw[4 * j + 1]),
                                   max((int)raw[4 * j + 2], (int)raw[4 * j + 3]));
        }
    };
    if (use_grammar) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            if constexpr (DT == SS_BF16) {
                const uint4 M = sh.gtab[gbits[j]];
                const uint32_t m4[4] = {M.x, M.y, M.z, M.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) raw[4 * j + k] = (raw[4 * j + k] & m4[k]) | (PAD & ~m4[k]);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t M = 0u - ((gbits[j] >> k) & 1u);
                    raw[4 * j + k] = (raw[4 * j + k] & M) | (PAD & ~M);
                }
            }
            chunk_max(j);
            __builtin_amdgcn_sched_barrier(0);   // chunks in arrival order
        }
    } else {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            chunk_max(j);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    int m;
    if constexpr (DT == SS_BF16) {
        s16x2 mm = bits_s16x2(cmx[0]);
#pragma unroll
        for (int j = 1; j < CPT; ++j) mm = __builtin_elementwise_max(mm, bits_s16x2(cmx[j]));
        m = max((int)mm.x, (int)mm.y);
    } else {
        m = (int)cmx[0];
#pragma unroll
        for (int j = 1; j < CPT; ++j) m = max(m, (int)cmx[j]);
    }

    // positive NaN anywhere in the tile -> general path; +inf of fp32 counts
    // as FLT_MAX for the threshold
    const int nan_floor = DT == SS_BF16 ? 0x7F80 : (int)F32_PINF_BITS;
    const bool special = m > nan_floor;
    if (DT == SS_F32) m = min(m, (int)F32_MAX_BITS);
    // at least 128 + nl tokens at or above tau, so that 128 remain once the
    // listed ones are set aside
    const bool nl_ok = nl_data <= S1_NL_FAST;
    const int kw = KMAX / S1_WAVES + (nl_ok ? (nl_data + S1_WAVES - 1) / S1_WAVES : 0);
    const int tau_w = wave_kth_largest<T::VAL_BITS>(m, kw);
    const uint64_t sp = __ballot(special);
    if (lane == 0) {
        sh.tau[wave] = tau_w;
        sh.special[wave] = sp != 0ull;
    }
    __syncthreads();   // tau
    int tau = sh.tau[0];
    bool any_special = false;
#pragma unroll
    for (int w = 0; w < S1_WAVES; ++w) {
        tau = min(tau, sh.tau[w]);
        any_special |= sh.special[w] != 0;
    }
    const bool fast = !any_special && tau >= 1 && nl_ok && P.aligned16;   // block-uniform

    if (fast) {
        // ---- chunks holding a value >= tau go to the wave's LDS area ----
        int wcnt = 0;
        const uint32_t T2 = ((uint32_t)(tau - 1) & 0xFFFFu) * 0x10001u;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            bool f;
            if constexpr (DT == SS_BF16)
                f = s16x2_bits(__builtin_elementwise_max(bits_s16x2(cmx[j]), bits_s16x2(T2))) != T2;
            else
                f = (int)cmx[j] >= tau;
            const uint64_t bal = __ballot(f);
            if (f && wcnt <= S1_CCAP) {   // slots up to S1_CCAP + 63 exist
                const int s = wcnt + lane_prefix(bal);
                sh.chunks[wave][s] = make_uint4(raw[4 * j], raw[4 * j + 1], raw[4 * j + 2], raw[4 * j + 3]);
                sh.cid[wave][s] = j * S1_THREADS + tid;
            }
            wcnt += __popcll(bal);
        }
        next();   // in.raw is free from here on
        wave_lds_sync();

        // ---- their elements >= tau that are not listed become keys, one
        // per lane per round ----
        const int nck = min(wcnt, S1_CCAP);
        int nk = 0;
        for (int s0 = 0; s0 < nck; s0 += WAVE) {
            const int s = s0 + lane;
            uint32_t sm = 0;
            int c = 0;
            if (s < nck) {
                c = sh.cid[wave][s];
                sm = chunk_survivors<DT>(sh.chunks[wave][s], tau);
                for (int i = 0; i < nl_data; ++i) {
                    const int2 e = sh.lcb[i];
                    if (e.x == c) sm &= ~(uint32_t)e.y;
                }
            }
            const auto elems = (const uint8_t*)&sh.chunks[wave][s < nck ? s : 0];
            for (;;) {
                const bool act = sm != 0;
                const uint64_t bal = __ballot(act);
                if (bal == 0ull) break;
                if (act) {
                    const int e = chunk_elem<DT>(__builtin_ctz(sm));
                    sm &= sm - 1u;
                    const int slot = nk + lane_prefix(bal);
                    const int local = c * EPC + e;
                    if (slot < S1_KCAP) {   // value > 0 and not NaN here
                        if constexpr (DT == SS_BF16) {
                            const uint32_t h = *(const uint16_t*)(elems + 2 * e);
                            sh.keys[wave][slot] = ((h | 0x8000u) << 16) | (0xFFFFu - (uint32_t)local);
                        } else {
                            const uint32_t h = *(const uint32_t*)(elems + 4 * e);
                            sh.keys[wave][slot] = key_f32(h, local, true, true);
                        }
                    }
                }
                nk += __popcll(bal);
            }
        }
        wave_lds_sync();
        if (wcnt > S1_CCAP || nk > S1_KCAP) {
            if (lane == 0) sh.ovf = 1;
        } else {
            const WList<Key> mine = wave_top128(sh.keys[wave], nk);
            sh.wl[wave][lane] = mine.lo;
            sh.wl[wave][lane + WAVE] = mine.hi;
        }
    } else {
        next();
    }
    __syncthreads();   // wave lists, ovf

    if (fast && sh.ovf == 0) {
        // ---- merge tree over the wave lists, in the lead wave's order
        // (lw = 0 is the lead): (0+1) on lw 0 and (2+3) on lw 1, then both ----
        const int lw = (wave - lead) & (S1_WAVES - 1);
        auto wl_of = [&](int l) -> WList<Key> {
            const int w = (l + lead) & (S1_WAVES - 1);
            return WList<Key>{sh.wl[w][lane], sh.wl[w][lane + WAVE]};
        };
        const int w2 = (lead + 2) & (S1_WAVES - 1);
        WList<Key> r{0, 0};
        if (lw < 2) {
            r = wave_merge(wl_of(2 * lw), wl_of(2 * lw + 1));
            if (lw == 1) {
                sh.wl[w2][lane] = r.lo;
                sh.wl[w2][lane + WAVE] = r.hi;
            }
        }
        __syncthreads();
        if (lw == 0) {
            r = wave_merge(r, WList<Key>{sh.wl[w2][lane], sh.wl[w2][lane + WAVE]});
            if (to_regs) {   // the caller takes the lead wave's registers
                *to_regs = r;
                return;
            }
            sh.surv[lane] = r.lo;
            sh.surv[lane + WAVE] = r.hi;
        }
        if (to_regs) return;
        __syncthreads();
        return;
    }

    // ---- general path: exact keys for every element (re-read from cache),
    // bisection for the 128th key.  The tile's listed tokens go to a bitmap
    // in LDS (over the chunk areas, no longer in use). ----
    uint32_t* lbm = (uint32_t*)&sh.chunks[0][0];
    static_assert(BN / 32 * 4 <= (int)sizeof(sh.chunks), "listed bitmap");
    for (int i = tid; i < BN / 32; i += S1_THREADS) lbm[i] = 0u;
    __syncthreads();
    for (int i = tid; i < nl; i += S1_THREADS) atomicOr(&lbm[sh.listed[i] >> 5], 1u << (sh.listed[i] & 31));
    __syncthreads();
    const auto gmask = gmem(P.aux.bitmask + (use_grammar ? (int64_t)row * P.aux.bitmask_stride : 0));
    auto ekey = [&](int q, int h) -> Key {
        const uint32_t d = load_dword(q);
        const int c = (q >> 2) * S1_THREADS + tid;
        const int e = DT == SS_BF16 ? 2 * (q & 3) + h : (q & 3);
        const int loc = c * EPC + e;
        const bool present = loc < nvalid && !((lbm[loc >> 5] >> (loc & 31)) & 1u);
        const bool allowed = present && (!use_grammar || ((gmask[(base + loc) >> 5] >> ((base + loc) & 31)) & 1u));
        if constexpr (DT == SS_BF16)
            return (Key)key_bf16(h ? (d >> 16) : (d & 0xFFFFu), loc, present, allowed);
        else
            return (Key)key_f32(d, loc, present, allowed);
    };
    constexpr int HALVES = DT == SS_BF16 ? 2 : 1;
    constexpr int KB = (int)sizeof(Key) * 8;
    Key res = 0;
    int parity = 0;
    for (int bit = KB - 1; bit >= 0; --bit) {
        const Key cand = res | ((Key)1 << bit);
        int c = 0;
#pragma nounroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int h = 0; h < HALVES; ++h) c += ekey(q, h) >= cand;
        c = wave_sum(c);
        if (lane == 0) sh.red[parity][wave] = c;
        __syncthreads();
        int tot = 0;
#pragma unroll
        for (int w = 0; w < S1_WAVES; ++w) tot += sh.red[parity][w];
        parity ^= 1;
        if (tot >= KMAX) res = cand;
    }
    const Key thr = res > (Key)1 ? res : (Key)1;   // key 0 = no token
    int cnt = 0;
#pragma nounroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int h = 0; h < HALVES; ++h) cnt += ekey(q, h) >= thr;
    int total;
    int off = block_excl_scan(cnt, sh.scan, &total);   // total <= 128 (keys are unique)
    Key* g = &sh.keys[0][0];
#pragma nounroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int h = 0; h < HALVES; ++h) {
            const Key k = ekey(q, h);
            if (k >= thr) g[off++] = k;
        }
    __syncthreads();
    if (wave == lead) {
        WList<Key> l{lane < total ? g[lane] : (Key)0, lane + WAVE < total ? g[lane + WAVE] : (Key)0};
        l = wave_sort128(l);
        if (to_regs) {
            *to_regs = l;
            return;
        }
        sh.surv[lane] = l.lo;
        sh.surv[lane + WAVE] = l.hi;
    }
    if (to_regs) return;
    __syncthreads();
}

// One tile, requested and processed in turn.  Without `to_regs` the sorted
// result is left in sh.surv behind a barrier; with it, the lead wave
// (s1_lead_wave) receives the result in registers and no wave waits at the
// end.
template <int DT>
__device__ __forceinline__ void stage1_tile(const Stage1Params& P, int row, int tile, S1Shared<DT>& sh,
                                            WList<typename S1Traits<DT>::Key>* to_regs = nullptr) {
    S1In<DT> in;
    tile_fetch<DT>(P, row, tile, in);
    tile_patch<DT>(P, row, tile, in);
    tile_process<DT>(P, row, tile, in, sh, [] {}, to_regs);
}

}  // namespace ssd
