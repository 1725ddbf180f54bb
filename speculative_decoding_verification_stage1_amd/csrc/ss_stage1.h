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
// Selection is exact, and on the common paths every element stays in
// registers after its one load.  Each lane holds 16 chunks of 16 bytes and takes the maximum of
// every chunk and of its whole slice; each wave finds the k-th largest of
// its 64 lane maxima, k = 32 + ceil(L/4) for L listed tokens still in the
// data, and the smallest of the four is a threshold tau with at least 128 +
// L tokens at or above it - so the 128 best unlisted tokens are all at or
// above tau.  Chunks whose maximum reaches tau (typically a few dozen per
// wave) are copied from registers to the wave's LDS area; each lane then
// takes one such chunk, and its elements >= tau that are not listed become
// keys, one per lane per round.  Each wave sorts its keys in registers, and
// a two-level merge tree gives the tile's 128.
//
// The comparisons run on one of two value forms held in the registers:
//   raw    the bit patterns read as signed integers; they order like the
//          floats only among positive values, so this form is used when
//          tau >= 1 (the usual case for logits);
//   order  the two's-complement order value v >= 0 ? v : -(v & magnitude)
//          of the bit pattern (bf16: per 16-bit half), which orders like
//          the floats over the whole range with -0 equal to +0; used when
//          the raw threshold is not positive (log-probabilities, sparse
//          grammars), with tau raised to the most negative finite value.
//          If fewer than 128 finite tokens remain (a grammar allowing few
//          tokens), the tile's remaining ranks are its -inf tokens (masked,
//          -inf or NaN) in id order.
// Masked tokens become all-ones patterns (a negative NaN: below any positive
// raw threshold, below -inf in the order form); elements past the end of V
// hold the smallest pattern.  Tiles with a positive NaN, or with more
// values tied near the threshold than the LDS areas hold, and rows that do
// not start on a 16-byte boundary take the exact path from memory
// (tile_exact_mem): the tile is read again, a radix select over LDS
// histograms finds the 128th value, and ties at it are taken in token
// order.
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
constexpr int S1_LIST_W = 2 * WAVE + SS_GAMMA_MAX;   // listed tokens one wave records: 64 prior, 64 bias, drafts
// listed tokens per tile left in the data (more are masked out): skipping
// them at the survivor step costs one LDS read per listed token and flagged
// chunk, the mask a fixed price per tile; measured on bf16 rows without a
// grammar, masking is faster from about ten per tile on, and no slower
// with five
constexpr int S1_NL_FAST = 4;

template <int DT> struct S1Traits;
template <> struct S1Traits<SS_BF16> {
    using Key = uint32_t;
    static constexpr int EPC = 8;                            // elements per chunk
    static constexpr int BN = EPC * S1_CPT * S1_THREADS;     // tile width 32768
    static constexpr int VAL_BITS = 16;                      // value range (int16)
    static constexpr int FINITE_MIN = -0x7F7F;               // order value of the most negative finite
    static constexpr int NINF_V = -0x7F80;                   // order value of -inf
    static constexpr int PINF_V = 0x7F80;                    // order value of +inf (kept: ranks above finite)
};
template <> struct S1Traits<SS_F32> {
    using Key = uint64_t;
    static constexpr int EPC = 4;
    static constexpr int BN = EPC * S1_CPT * S1_THREADS;     // 16384
    static constexpr int VAL_BITS = 32;
    static constexpr int FINITE_MIN = -0x7F7FFFFF;
    static constexpr int NINF_V = -0x7F800000;
    static constexpr int PINF_V = 0x7F7FFFFF;                // +inf counts as FLT_MAX
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

// Two's-complement order value of a raw pattern (bf16: of each 16-bit
// half): v >= 0 ? v : -(v & magnitude).  Monotone in the float value, with
// -0 and +0 equal.
template <int DT>
__device__ __forceinline__ uint32_t order_value(uint32_t x) {
    if constexpr (DT == SS_BF16) {
        const s16x2 s = bits_s16x2(x) >> (s16x2){15, 15};   // -1 on negative halves
        const s16x2 t = bits_s16x2(x & 0x7FFF7FFFu) ^ s;
        return s16x2_bits(t - s);
    } else {
        const int32_t s = (int32_t)x >> 31;
        return (uint32_t)((((int32_t)(x & 0x7FFFFFFFu)) ^ s) - s);
    }
}

// Packed key of a present element from its (finite or +inf) value in either
// register form - a positive raw pattern is its own order value - and its
// index in the tile.
template <int DT>
__device__ __forceinline__ typename S1Traits<DT>::Key value_key(int v, int local) {
    if constexpr (DT == SS_BF16) {
        const uint32_t k16 = (uint32_t)(v + 0x8000 - (v < 0 ? 1 : 0));
        return (k16 << 16) | (0xFFFFu - (uint32_t)local);
    } else {
        const uint32_t k32 = (uint32_t)min(v, S1Traits<SS_F32>::PINF_V) + 0x80000000u - (v < 0 ? 1u : 0u);
        return ((uint64_t)k32 << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)local);
    }
}
template <int DT>
__device__ __forceinline__ typename S1Traits<DT>::Key ninf_key(int local) {
    return value_key<DT>(S1Traits<DT>::NINF_V, local);
}

template <int DT>
struct S1Shared {
    using Key = typename S1Traits<DT>::Key;
    uint4 chunks[S1_WAVES][S1_CCAP + WAVE];   // flagged chunks, per wave (fast path); exact path: bitmap
    int cid[S1_WAVES][S1_CCAP + WAVE];        // their chunk index in the tile
    Key keys[S1_WAVES][S1_KCAP];       // survivors per wave (fast path); exact path: flat
    Key wl[S1_WAVES][KMAX];            // per-wave sorted lists
    Key surv[KMAX];                    // result: the tile's 128 best, sorted; -inf ranks of sparse tiles
    uint4 gtab[256];                   // bf16 masks: dword keep masks of a chunk by its allowed byte
    uint32_t gmw[S1Traits<DT>::BN / 32];   // the tile's mask (grammar and/or listed tokens)
    int listed[S1_WAVES][S1_LIST_W];   // tile-local index of each listed token, per recording wave
    int2 lcb[S1_WAVES][S1_LIST_W];     // its chunk, and its bit in a chunk's survivor mask
    alignas(16) int nlw[S1_WAVES];
    int tau[S1_WAVES];
    int tau2[S1_WAVES];
    int special[S1_WAVES];
    int nk[S1_WAVES];
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
// Elements of a chunk whose value (in its register form) is >= tau.
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
    int l_pid, l_pct, l_bid;    // entries 64lw .. 64lw+63 of the request's lists (lw: wave after the lead)
    int l_did;                  // lead wave: draft `lane` of the request (verification), or -1
    uint32_t rq_flags, rq_lists; // the request's flags and its n_prior | n_bias << 16
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
    (void)wave; (void)lead; (void)lane; (void)b; (void)vec; (void)NQ; (void)PAD; (void)full;

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
    // the wave lw places after the lead (lw = 0: the lead): entries 64lw ..
    // 64lw+63 of the request's lists
    in.l_pid = -1;
    in.l_pct = 0;
    in.l_bid = -1;
    {
        const int j0 = ((wave - lead) & (S1_WAVES - 1)) * WAVE;   // wave-uniform
        const int j = j0 + lane;
        if (P.aux.prior_ids && P.aux.prior_cnt && j0 < P.aux.prior_stride && j < P.aux.prior_stride) {
            const int64_t o = (int64_t)b * P.aux.prior_stride + j;
            in.l_pid = gmem(P.aux.prior_ids)[o];
            in.l_pct = gmem(P.aux.prior_cnt)[o];
        }
        if (P.aux.bias_ids && j0 < P.aux.bias_stride && j < P.aux.bias_stride)
            in.l_bid = gmem(P.aux.bias_ids)[(int64_t)b * P.aux.bias_stride + j];
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
        in.rq_flags = rq[0] & 0xFFFFu;   // the 16-bit flags (top_k above them)
        in.rq_lists = rq[2];              // n_prior | n_bias << 16
    }
}

// Tiles that are not whole 16-byte chunks of an aligned row: chunks not
// wholly inside V become PAD, and the one that straddles the end is
// completed by its owner thread from the elements inside V.  Waits for the
// tile's loads, so full aligned tiles skip it.  (Rows that do not start on
// a 16-byte boundary load nothing here: the exact path reads them.)
template <int DT>
__device__ __forceinline__ void tile_patch(const Stage1Params& P, int row, int tile, S1In<DT>& in) {
    S1_TILE_GEOMETRY
    if (vec) return;
    if (!P.aligned16) return;   // read by the exact path instead
    const int cp = nvalid / EPC;   // first chunk not wholly inside V
#pragma unroll
    for (int j = 0; j < CPT; ++j)
        if (j * S1_THREADS + tid >= cp) {
#pragma unroll
            for (int k = 0; k < 4; ++k) in.raw[4 * j + k] = PAD;
        }
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

// Keep masks of this thread's chunk j from an LDS bitmap laid out like the
// grammar bitmask (bit e of byte c: element e of chunk c): per dword, all
// ones on the elements whose bit is set (clear, with `invert`).  bf16 goes
// through the 256-entry table of dword masks.
template <int DT>
__device__ __forceinline__ uint4 chunk_keep(const S1Shared<DT>& sh, const uint32_t* bm, int j, bool invert) {
    const uint8_t* by = (const uint8_t*)bm;
    const int c = j * S1_THREADS + (int)threadIdx.x;
    if constexpr (DT == SS_BF16) {
        const uint32_t g = by[c] ^ (invert ? 0xFFu : 0u);
        return sh.gtab[g];
    } else {
        const uint32_t g = ((uint32_t)by[c >> 1] >> ((c & 1) * 4)) ^ (invert ? 0xFu : 0u);
        return make_uint4(0u - (g & 1u), 0u - ((g >> 1) & 1u), 0u - ((g >> 2) & 1u), 0u - ((g >> 3) & 1u));
    }
}

// chunk_keep from the bitmap byte alone, without the table (the rarely
// taken paths use it: table reads there cost the kernel registers).
template <int DT>
__device__ __forceinline__ uint4 chunk_keep_alu(const uint32_t* bm, int j, bool invert) {
    const uint8_t* by = (const uint8_t*)bm;
    const int c = j * S1_THREADS + (int)threadIdx.x;
    if constexpr (DT == SS_BF16) {
        const uint32_t g = by[c] ^ (invert ? 0xFFu : 0u);
        uint32_t mk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            mk[k] = ((0u - ((g >> (2 * k)) & 1u)) & 0x0000FFFFu) | ((0u - ((g >> (2 * k + 1)) & 1u)) & 0xFFFF0000u);
        return make_uint4(mk[0], mk[1], mk[2], mk[3]);
    } else {
        const uint32_t g = ((uint32_t)by[c >> 1] >> ((c & 1) * 4)) ^ (invert ? 0xFu : 0u);
        return make_uint4(0u - (g & 1u), 0u - ((g >> 1) & 1u), 0u - ((g >> 2) & 1u), 0u - ((g >> 3) & 1u));
    }
}

// Elements of a ragged tile past the end of V take PAD (any register form).
template <int DT>
__device__ __forceinline__ void pad_absent(uint32_t (&raw)[S1_CPT * 4], int nvalid) {
    constexpr int EPC = S1Traits<DT>::EPC;
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < S1_CPT; ++j) {
        const int n = nvalid - (j * S1_THREADS + tid) * EPC;   // elements of the chunk inside V
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if constexpr (DT == SS_BF16) {
                const uint32_t keep = (2 * k < n ? 0x0000FFFFu : 0u) | (2 * k + 1 < n ? 0xFFFF0000u : 0u);
                raw[4 * j + k] = (raw[4 * j + k] & keep) | (0x80008000u & ~keep);
            } else {
                raw[4 * j + k] = k < n ? raw[4 * j + k] : 0x80000000u;
            }
        }
    }
}

// Maximum of chunk j (signed, per half for bf16 then both halves).
template <int DT>
__device__ __forceinline__ uint32_t chunk_max(const uint32_t (&raw)[S1_CPT * 4], int j) {
    if constexpr (DT == SS_BF16) {
        const s16x2 a = __builtin_elementwise_max(bits_s16x2(raw[4 * j]), bits_s16x2(raw[4 * j + 1]));
        const s16x2 c = __builtin_elementwise_max(bits_s16x2(raw[4 * j + 2]), bits_s16x2(raw[4 * j + 3]));
        return s16x2_bits(__builtin_elementwise_max(a, c));
    } else {
        return (uint32_t)max(max((int)raw[4 * j], (int)raw[4 * j + 1]), max((int)raw[4 * j + 2], (int)raw[4 * j + 3]));
    }
}
// Largest value of the lane (signed); `clamp`: fp32 +inf counts as FLT_MAX.
template <int DT>
__device__ __forceinline__ int lane_max(const uint32_t (&cmx)[S1_CPT], bool clamp) {
    if constexpr (DT == SS_BF16) {
        s16x2 mm = bits_s16x2(cmx[0]);
#pragma unroll
        for (int j = 1; j < S1_CPT; ++j) mm = __builtin_elementwise_max(mm, bits_s16x2(cmx[j]));
        return max((int)mm.x, (int)mm.y);
    } else {
        int m = (int)cmx[0];
#pragma unroll
        for (int j = 1; j < S1_CPT; ++j) m = max(m, (int)cmx[j]);
        return clamp ? min(m, (int)F32_MAX_BITS) : m;
    }
}

// The tile's tokens left out of the selection, as a bitmap over the tile
// (bit (i & 31) of word i >> 5): its listed tokens and the elements past V.
// Written over the chunk areas; ends with a barrier.
template <int DT>
__device__ __forceinline__ uint32_t* exclusion_bitmap(S1Shared<DT>& sh, int nvalid) {
    constexpr int BN = S1Traits<DT>::BN;
    static_assert(BN / 32 * 4 <= (int)sizeof(sh.chunks), "exclusion bitmap");
    uint32_t* ebm = (uint32_t*)&sh.chunks[0][0];
    for (int i = threadIdx.x; i < BN / 32; i += S1_THREADS) {
        const int lo = i * 32;
        ebm[i] = lo + 32 <= nvalid ? 0u : (lo >= nvalid ? ~0u : ~((1u << (nvalid - lo)) - 1u));
    }
    __syncthreads();
    for (int w = 0; w < S1_WAVES; ++w)
        for (int i = threadIdx.x; i < sh.nlw[w]; i += S1_THREADS)
            atomicOr(&ebm[sh.listed[w][i] >> 5], 1u << (sh.listed[w][i] & 31));
    __syncthreads();
    return ebm;
}

// Chunks holding a value >= tau (register form of `raw`, chunk maxima
// `cmx`) go to the wave's LDS area; their elements >= tau that are not
// among the nl_data listed tokens become keys, one per lane per round; each
// wave's best 128 go to sh.wl[wave], its survivor count to sh.nk[wave], and
// sh.ovf is set when a wave has more chunks or survivors than its areas
// hold.  No barrier.
template <int DT>
__device__ __forceinline__ void select_ge(const uint32_t (&raw)[S1_CPT * 4], const uint32_t (&cmx)[S1_CPT], int tau,
                                          int nl_data, S1Shared<DT>& sh) {
    using Key = typename S1Traits<DT>::Key;
    constexpr int EPC = S1Traits<DT>::EPC;
    const int tid = threadIdx.x;
    const int wave = tid / WAVE;
    const int lane = lane_id();
    int wcnt = 0;
    const uint32_t T2 = ((uint32_t)(tau - 1) & 0xFFFFu) * 0x10001u;
#pragma unroll
    for (int j = 0; j < S1_CPT; ++j) {
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
    wave_lds_sync();
    const int nck = min(wcnt, S1_CCAP);
    int nk = 0;
    for (int s0 = 0; s0 < nck; s0 += WAVE) {
        const int s = s0 + lane;
        uint32_t sm = 0;
        int c = 0;
        if (s < nck) {
            c = sh.cid[wave][s];
            sm = chunk_survivors<DT>(sh.chunks[wave][s], tau);
            if (nl_data > 0)
                for (int w = 0; w < S1_WAVES; ++w)
                    for (int i = 0; i < sh.nlw[w]; ++i) {
                        const int2 e = sh.lcb[w][i];
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
                if (slot < S1_KCAP) {   // a finite value (or +inf) here
                    int v;
                    if constexpr (DT == SS_BF16) v = (int)*(const short*)(elems + 2 * e);
                    else v = *(const int*)(elems + 4 * e);
                    sh.keys[wave][slot] = value_key<DT>(v, local);
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
    if (lane == 0) sh.nk[wave] = nk;
}

// Merge tree over the four wave lists, in the lead wave's order (lw = 0 is
// the lead): (0+1) on lw 0 and (2+3) on lw 1, then both.  One barrier; the
// result is valid in the lead wave.
template <int DT>
__device__ __forceinline__ WList<typename S1Traits<DT>::Key> merge_lists(S1Shared<DT>& sh) {
    using Key = typename S1Traits<DT>::Key;
    const int wave = threadIdx.x / WAVE;
    const int lane = lane_id();
    const int lead = s1_lead_wave();
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
    if (lw == 0) r = wave_merge(r, WList<Key>{sh.wl[w2][lane], sh.wl[w2][lane + WAVE]});
    return r;
}

// Exact path for the tiles the threshold select cannot take (a positive
// NaN, or more values tied near the threshold than its LDS areas hold):
// the tile is read again from memory, element by element, thread t taking
// tile indices [t*BN/256, (t+1)*BN/256), so that thread order is token
// order.  Each element's canonical order value: -inf for masked tokens and
// NaN, +inf as FLT_MAX for fp32; tokens left out (listed, past V: set in
// the LDS bitmap `ebm`) are skipped.  A radix select on the order key, 8
// bits per pass over an LDS histogram, finds the 128th largest value T;
// every token above T is kept (fewer than 128), and the first 128 - #{> T}
// tokens equal to T in token order (a block scan of per-thread counts).
// The keys are sorted by the lead wave into sh.surv.  Not inlined: the
// common path keeps the tile in registers and this path must not add to
// them.  Ends with a barrier.
template <int DT>
__device__ __attribute__((noinline)) void tile_exact_mem(const char* rowp, int nvalid, bool use_mask, bool aligned,
                                                          S1Shared<DT>& shg, const uint32_t* ebm_g) {
    using TT = S1Traits<DT>;
    using Key = typename TT::Key;
    constexpr int EPC = TT::EPC;                    // elements per 16-byte chunk
    constexpr int CPT = TT::BN / EPC / S1_THREADS;  // chunks per thread
    const int tid = threadIdx.x;
    const int wave = tid / WAVE;
    const int lane = lane_id();
    // The LDS arrays with their address space spelled out: this function is
    // not inlined, so `shg` arrives as a generic pointer, and generic
    // accesses would have to wait for every global load in flight.
    using L32 = __attribute__((address_space(3))) uint32_t;
    using LI = __attribute__((address_space(3))) int;
    using LK = __attribute__((address_space(3))) Key;
    const L32* ebm = (const L32*)ebm_g;
    const L32* gmw = (const L32*)shg.gmw;
    LI* hist = (LI*)&shg.cid[0][0];
    static_assert(sizeof(shg.cid) >= 256 * sizeof(int), "histogram");
    LI* ctr = (LI*)&shg.red[0][0];
    LK* g = (LK*)&shg.keys[0][0];
    const int nfull = aligned ? nvalid / EPC : 0;   // chunks read with one 16-byte load
    // chunk c's data as four dwords (element e of a bf16 chunk: half e & 1
    // of dword e >> 1); elements past the end read as zero
    auto load = [&](int c, uint32_t (&w)[4]) {
        if (c < nfull) {
            const vu32x4 d = gmem((const vu32x4*)rowp)[c];
            w[0] = d.x;
            w[1] = d.y;
            w[2] = d.z;
            w[3] = d.w;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) w[k] = 0u;
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                const int i = c * EPC + e;
                if (i >= nvalid) continue;
                if constexpr (DT == SS_BF16) w[e >> 1] |= (uint32_t)gmem((const uint16_t*)rowp)[i] << (16 * (e & 1));
                else w[e] = gmem((const uint32_t*)rowp)[i];
            }
        }
    };
    // f(i, u, v) for every token of chunk c that is not left out: u its
    // unsigned order key (larger = better), v its order value
    auto chunk_keys = [&](int c, const uint32_t (&w)[4], auto&& f) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
            const int i = c * EPC + e;
            if (i >= nvalid || ((ebm[i >> 5] >> (i & 31)) & 1u)) continue;
            const bool masked = use_mask && !((gmw[i >> 5] >> (i & 31)) & 1u);
            int v;
            uint32_t u;
            if constexpr (DT == SS_BF16) {
                const uint32_t h = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                const bool nan = (h & 0x7FFFu) > 0x7F80u;
                v = (h & 0x8000u) ? -(int)(h & 0x7FFFu) : (int)h;
                if (masked || nan) v = TT::NINF_V;
                u = (uint32_t)(v + 0x8000);
            } else {
                const uint32_t x = w[e];
                const bool nan = (x & 0x7FFFFFFFu) > 0x7F800000u;
                v = (x & 0x80000000u) ? -(int)(x & 0x7FFFFFFFu) : (int)x;
                v = min(v, TT::PINF_V);
                if (masked || nan) v = TT::NINF_V;
                u = (uint32_t)v ^ 0x80000000u;
            }
            f(i, u, v);
        }
    };
    // chunks chunk_of(0 .. CPT-1), their loads issued in batches of eight
    // before any is used
    constexpr int BATCH = 8;
    static_assert(CPT % BATCH == 0, "batches");
    auto chunks = [&](auto&& chunk_of, auto&& f) {
        for (int k0 = 0; k0 < CPT; k0 += BATCH) {
            uint32_t w[BATCH][4];
#pragma unroll
            for (int b = 0; b < BATCH; ++b) load(chunk_of(k0 + b), w[b]);
#pragma unroll
            for (int b = 0; b < BATCH; ++b) chunk_keys(chunk_of(k0 + b), w[b], f);
        }
    };
    // the tile in coalesced order (chunk k * 256 + tid), for the passes
    // whose order does not matter
    auto tile_pass = [&](auto&& f) { chunks([&](int k) { return k * S1_THREADS + tid; }, f); };
    constexpr int KBITS = DT == SS_BF16 ? 16 : 32;
    uint32_t prefix = 0;   // the digits of T's key found so far
    int kneed = KMAX;      // how many of the tokens with this prefix are still wanted
    int n_all = 0;
    bool take_all = false;
    for (int shift = KBITS - 8; shift >= 0; shift -= 8) {   // block-uniform
        hist[tid] = 0;
        __syncthreads();
        tile_pass([&](int, uint32_t u, int) {
            if (shift + 8 >= KBITS || (u >> (shift + 8)) == prefix)
                __hip_atomic_fetch_add(&hist[(u >> shift) & 255u], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        });
        __syncthreads();
        // the digit b of the kneed-th largest: lane l sums bins 4l..4l+3,
        // suffix sums from the top give the lane, then its bins
        int s4[4], s = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            s4[k] = hist[4 * lane + k];
            s += s4[k];
        }
        const int pre = wave_incl_scan(s);
        const int tot = __shfl(pre, WAVE - 1, WAVE);
        const int suffix = tot - pre + s;   // bins 4*lane .. 255
        if (shift == KBITS - 8) {
            n_all = __builtin_amdgcn_readfirstlane(tot);
            if (n_all <= KMAX) {   // the tile holds no more than 128 tokens: all of them
                take_all = true;
                break;
            }
        }
        const uint64_t ok = __ballot(suffix >= kneed);
        const int L = 63 - __builtin_clzll(ok);   // highest lane whose suffix reaches kneed
        const int above = __shfl(suffix - s, L, WAVE);   // bins above lane L's
        int b = 4 * L + 3, acc = above;
        const int h3 = __shfl(s4[3], L, WAVE), h2 = __shfl(s4[2], L, WAVE);
        const int h1 = __shfl(s4[1], L, WAVE);
        if (acc + h3 >= kneed) b = 4 * L + 3;
        else if (acc + h3 + h2 >= kneed) { b = 4 * L + 2; acc += h3; }
        else if (acc + h3 + h2 + h1 >= kneed) { b = 4 * L + 1; acc += h3 + h2; }
        else { b = 4 * L; acc += h3 + h2 + h1; }
        kneed -= __builtin_amdgcn_readfirstlane(acc);
        prefix = (prefix << 8) | (uint32_t)__builtin_amdgcn_readfirstlane(b);
        __syncthreads();   // the histogram is read before the next pass clears it
    }
    // T's key is `prefix`; `kneed` tokens equal to T are wanted
    if (tid == 0) *ctr = 0;
    __syncthreads();
    const int n_gt = KMAX - kneed;
    tile_pass([&](int i, uint32_t u, int v) {
        if (take_all || u > prefix)
            g[__hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)] = value_key<DT>(v, i);
    });
    // ties at T in token order: thread t owns the contiguous chunks
    // t * CPT .. t * CPT + CPT - 1
    auto own = [&](int k) { return tid * CPT + k; };
    int nties = 0;
    if (!take_all) chunks(own, [&](int, uint32_t u, int) { nties += u == prefix; });
    int total;
    int r = block_excl_scan(take_all ? 0 : nties, (int*)shg.scan, &total);   // ties before this thread's
    if (!take_all && r < kneed)
        chunks(own, [&](int i, uint32_t u, int v) {
            if (u == prefix && r < kneed) g[n_gt + r++] = value_key<DT>(v, i);
        });
    __syncthreads();
    const int n = take_all ? n_all : KMAX;
    if (wave == s1_lead_wave()) {
        WList<Key> l{lane < n ? g[lane] : (Key)0, lane + WAVE < n ? g[lane + WAVE] : (Key)0};
        l = wave_sort128(l);
        shg.surv[lane] = l.lo;
        shg.surv[lane + WAVE] = l.hi;
    }
    __syncthreads();
}

// The 128 best tokens of tile `tile` of row `row` (whose data `in` holds),
// sorted best first (key 0 = no token): left in sh.surv[0..128) behind a
// final barrier, or, with `to_regs`, handed to the lead wave's registers
// with no final barrier (the other waves return early).
template <int DT>
__device__ __forceinline__ void tile_process(const Stage1Params& P, int row, int tile, S1In<DT>& in,
                                             S1Shared<DT>& sh, WList<typename S1Traits<DT>::Key>* to_regs = nullptr) {
    S1_TILE_GEOMETRY
    using Key = typename T::Key;
    static_assert(S1_WAVES == 4, "merge tree");
    uint32_t(&raw)[NQ] = in.raw;

    const uint32_t flags = __builtin_amdgcn_readfirstlane(in.rq_flags);
    const uint32_t lists = __builtin_amdgcn_readfirstlane(in.rq_lists);
    // a list longer than its stride or its limit makes the row invalid
    // (reported by Stage 2); the tiles then use no list at all
    const int np_all = (int)(lists & 0xFFFFu), nb_all = (int)(lists >> 16);
    const int n_prior = np_all <= P.aux.prior_stride && np_all <= SS_PRIOR_MAX ? np_all : 0;
    const int n_bias = nb_all <= P.aux.bias_stride && nb_all <= SS_BIAS_MAX ? nb_all : 0;
    const bool use_grammar = (flags & SS_GRAMMAR) && P.aux.bitmask;
    const bool use_prior = (flags & (SS_REP | SS_FREQPRES)) && P.aux.prior_ids && P.aux.prior_cnt && n_prior > 0;
    const bool use_bias = (flags & SS_BIAS) && P.aux.bias_ids && n_bias > 0;

    // the 256-entry table of dword keep masks (bf16): entry g sets the low
    // half of dword k when bit 2k of g is set, the high half for bit 2k + 1
    auto build_gtab = [&] {
        if constexpr (DT == SS_BF16) {
            uint32_t mk[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                mk[k] = (((uint32_t)tid >> (2 * k)) & 1u ? 0x0000FFFFu : 0u) |
                        (((uint32_t)tid >> (2 * k + 1)) & 1u ? 0xFFFF0000u : 0u);
            sh.gtab[tid] = make_uint4(mk[0], mk[1], mk[2], mk[3]);
        }
    };
    // the tile's grammar words go to LDS; each thread then reads the bits
    // of its own chunks
    if (use_grammar) {
#pragma unroll
        for (int k = 0; k < CPT * EPC / 32; ++k) sh.gmw[tid + k * S1_THREADS] = in.gw[k];
        build_gtab();
    }
    const int l_pid = in.l_pid, l_pct = in.l_pct, l_bid = in.l_bid;

    // ---- tokens of this tile named by an active list (ranked in Stage 2,
    // left out here): the wave lw places after the lead records list
    // entries 64lw .. 64lw+63, the lead wave also the earlier drafts; the
    // entries past the first 256 of a longer list go straight into the
    // mask below ----
    const int lw = (wave - lead) & (S1_WAVES - 1);
    const bool has_slice = (use_prior && n_prior > lw * WAVE) || (use_bias && n_bias > lw * WAVE) || wave == lead;
    if (has_slice) {   // wave-uniform
        int nl = 0;
        int* const lst = sh.listed[wave];
        int2* const lcbw = sh.lcb[wave];
        auto record = [&](bool ok, int loc) {
            const uint64_t bal = __ballot(ok);
            if (ok) {
                const int i = nl + lane_prefix(bal);
                lst[i] = loc;
                lcbw[i] = make_int2(loc / EPC, (int)chunk_bit<DT>(loc % EPC));
            }
            nl += __popcll(bal);
        };
        const int j = lw * WAVE + lane;
        if (use_prior) {
            const int loc = l_pid - base;
            record(j < n_prior && l_pct >= 1 && l_pid >= 0 && l_pid < P.V && loc >= 0 && loc < nvalid, loc);
        }
        if (use_bias) {
            const int loc = l_bid - base;
            record(j < n_bias && l_bid >= 0 && l_bid < P.V && loc >= 0 && loc < nvalid, loc);
        }
        // earlier drafts in the penalty history (verification)
        const int nh = wave == lead ? draft_hist_len(P, flags, row) : 0;
        if (nh > 0) {
            const int loc = in.l_did - base;
            record(lane < nh && in.l_did >= 0 && in.l_did < P.V && loc >= 0 && loc < nvalid, loc);
        }
        if (lane == 0) {
            sh.nlw[wave] = nl;
            if (wave == lead) sh.ovf = 0;
        }
    } else if (lane == 0) {
        sh.nlw[wave] = 0;
    }
    __syncthreads();   // listed tokens, grammar table
    const int4 nl4 = *(const int4*)sh.nlw;   // one read
    const int nl = __builtin_amdgcn_readfirstlane(nl4.x + nl4.y + nl4.z + nl4.w);
    // The tile's listed tokens are cleared from the mask when the row has a
    // grammar mask, or when there are more than S1_NL_FAST of them (each
    // wave keeps a quarter of those left in the data as extra candidates,
    // which lowers the threshold, and the survivor step skips them one by
    // one): the mask then leaves them out like any disallowed token,
    // and the threshold and survivor steps need not know about them.
    const bool long_lists = (use_prior && n_prior > S1_WAVES * WAVE) || (use_bias && n_bias > S1_WAVES * WAVE);
    const bool fold = (nl > 0 && (use_grammar || nl > S1_NL_FAST)) || long_lists;   // block-uniform
    const bool use_mask = use_grammar || fold;
    if (fold) {
        if (!use_grammar) {   // an all-ones mask to clear them from
            for (int i = tid; i < BN / 32; i += S1_THREADS) sh.gmw[i] = ~0u;
            build_gtab();
            __syncthreads();
        }
        const int nlv[S1_WAVES] = {nl4.x, nl4.y, nl4.z, nl4.w};
#pragma unroll
        for (int w = 0; w < S1_WAVES; ++w)
            for (int i = tid; i < nlv[w]; i += S1_THREADS) {
                const int loc = sh.listed[w][i];
                atomicAnd(&sh.gmw[loc >> 5], ~(1u << (loc & 31)));
            }
        if (long_lists) {   // the entries past the recorded 256
            const int64_t ob = (int64_t)b * P.aux.prior_stride, obb = (int64_t)b * P.aux.bias_stride;
            for (int j = S1_WAVES * WAVE + tid; use_prior && j < n_prior; j += S1_THREADS) {
                const int id = gmem(P.aux.prior_ids)[ob + j], loc = id - base;
                if (gmem(P.aux.prior_cnt)[ob + j] >= 1 && id >= 0 && id < P.V && loc >= 0 && loc < nvalid)
                    atomicAnd(&sh.gmw[loc >> 5], ~(1u << (loc & 31)));
            }
            for (int j = S1_WAVES * WAVE + tid; use_bias && j < n_bias; j += S1_THREADS) {
                const int id = gmem(P.aux.bias_ids)[obb + j], loc = id - base;
                if (id >= 0 && id < P.V && loc >= 0 && loc < nvalid) atomicAnd(&sh.gmw[loc >> 5], ~(1u << (loc & 31)));
            }
        }
        __syncthreads();
    }
    const int nl_data = fold ? 0 : nl;   // listed tokens still present in the data (<= 128)
    WList<Key> r{0, 0};
    auto exact = [&] {   // the exact path, from memory (sh.surv, then the lead wave's registers)
        const uint32_t* ebm = exclusion_bitmap<DT>(sh, nvalid);
        tile_exact_mem<DT>(rowp, nvalid, use_mask, P.aligned16 != 0, sh, ebm);
        if (wave == lead) r = WList<Key>{sh.surv[lane], sh.surv[lane + WAVE]};
    };
    auto finish = [&] {
        if (wave == lead) {
            if (to_regs) {   // the caller takes the lead wave's registers
                *to_regs = r;
                return;
            }
            sh.surv[lane] = r.lo;
            sh.surv[lane + WAVE] = r.hi;
        }
        if (to_regs) return;
        __syncthreads();
    };
    if (!P.aligned16) {   // rows not on a 16-byte boundary (block-uniform)
        exact();
        finish();
        return;
    }

    // ---- mask and maxima per chunk and per lane (raw patterns read as
    // signed), chunk by chunk in the order the loads were issued, so that
    // each waits only for its own data.  A masked element becomes all ones,
    // a negative NaN: below any positive threshold in the raw form, below
    // -inf in the order form, and -inf in the exact path, as the mask asks ----
    uint32_t cmx[CPT];
    if (use_mask) {
        // every chunk's mask byte first (independent reads), then one table
        // read per chunk in arrival order
        uint32_t gbits[CPT];
        const uint8_t* gb = (const uint8_t*)sh.gmw;
#pragma unroll
        for (int j = 0; j < CPT; ++j)
            gbits[j] = DT == SS_BF16 ? gb[j * S1_THREADS + tid]
                                     : (uint32_t)gb[(j * S1_THREADS + tid) >> 1] >> ((tid & 1) * 4);
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            uint4 M;
            if constexpr (DT == SS_BF16) {
                M = sh.gtab[gbits[j]];
            } else {
                const uint32_t g = gbits[j];
                M = make_uint4(0u - (g & 1u), 0u - ((g >> 1) & 1u), 0u - ((g >> 2) & 1u), 0u - ((g >> 3) & 1u));
            }
            const uint32_t m4[4] = {M.x, M.y, M.z, M.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) raw[4 * j + k] |= ~m4[k];   // masked: all ones
            cmx[j] = chunk_max<DT>(raw, j);
            __builtin_amdgcn_sched_barrier(0);   // chunks in arrival order
        }
    } else {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            cmx[j] = chunk_max<DT>(raw, j);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // a positive NaN (the largest signed patterns) sends the tile to the
    // exact path; fp32 +inf counts as FLT_MAX for the threshold
    const int mraw = lane_max<DT>(cmx, false);
    const bool special = mraw > (DT == SS_BF16 ? 0x7F80 : (int)F32_PINF_BITS);
    int m = DT == SS_F32 ? min(mraw, (int)F32_MAX_BITS) : mraw;
    // at least 128 + nl tokens at or above tau, so that 128 remain once the
    // listed ones are set aside
    const int kw = KMAX / S1_WAVES + (nl_data + S1_WAVES - 1) / S1_WAVES;
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
    // block-uniform: raw form (tau >= 1), order form, or the exact path
    tau = __builtin_amdgcn_readfirstlane(tau);
    any_special = __builtin_amdgcn_readfirstlane((int)any_special) != 0;
    const bool ordered = !any_special && tau < 1;
    if (ordered) {
        // the order form (masked elements fall below -inf by themselves);
        // elements past V back to PAD
#pragma unroll
        for (int q = 0; q < NQ; ++q) raw[q] = order_value<DT>(raw[q]);
        if (!full) pad_absent<DT>(raw, nvalid);
#pragma unroll
        for (int j = 0; j < CPT; ++j) cmx[j] = chunk_max<DT>(raw, j);
        m = lane_max<DT>(cmx, true);
        const int t2 = wave_kth_largest<T::VAL_BITS>(m, kw);
        if (lane == 0) sh.tau2[wave] = t2;
        __syncthreads();
        tau = sh.tau2[0];
#pragma unroll
        for (int w = 1; w < S1_WAVES; ++w) tau = min(tau, sh.tau2[w]);
        tau = __builtin_amdgcn_readfirstlane(max(tau, T::FINITE_MIN));   // below it: -inf, NaN, masked
    }

    if (!any_special) select_ge<DT>(raw, cmx, tau, nl_data, sh);
    __syncthreads();   // wave lists, ovf, survivor counts

    if (!any_special && __builtin_amdgcn_readfirstlane(sh.ovf) == 0) {
        // survivors in all: fewer than 128 only in the order form (the finite
        // tokens of a tile whose grammar allows few); the remaining ranks are
        // the tile's -inf tokens in token order, found among its first
        // S1_THREADS chunks (the first 128 + listed + finite indices lie there)
        const int n_fin = ordered ? __builtin_amdgcn_readfirstlane(sh.nk[0] + sh.nk[1] + sh.nk[2] + sh.nk[3]) : KMAX;
        const bool fill = n_fin < KMAX;   // block-uniform; only in the order form
        if (fill) {
            if (tid < KMAX && tid >= n_fin) sh.surv[tid] = (Key)0;
            const uint32_t* ebm = exclusion_bitmap<DT>(sh, nvalid);
            const uint4 E = chunk_keep_alu<DT>(ebm, 0, true);   // chunk tid: tile indices tid*EPC ..
            const uint32_t e4[4] = {E.x, E.y, E.z, E.w};
            uint32_t fm = 0;   // bit e: element e is a -inf token
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (DT == SS_BF16) {
                    const int lo16 = (int)(short)(raw[k] & 0xFFFFu), hi16 = (int)(short)(raw[k] >> 16);
                    fm |= ((lo16 < T::FINITE_MIN && (e4[k] & 0xFFFFu)) ? 1u : 0u) << (2 * k);
                    fm |= ((hi16 < T::FINITE_MIN && (e4[k] >> 16)) ? 1u : 0u) << (2 * k + 1);
                } else {
                    fm |= (((int)raw[k] < T::FINITE_MIN && e4[k]) ? 1u : 0u) << k;
                }
            }
            int tot;
            int rk = n_fin + block_excl_scan(__builtin_popcount(fm), sh.scan, &tot);
            while (fm) {
                const int e = __builtin_ctz(fm);
                fm &= fm - 1u;
                if (rk < KMAX) sh.surv[rk] = ninf_key<DT>(tid * EPC + e);
                ++rk;
            }
            __syncthreads();
        }
        r = merge_lists<DT>(sh);
        if (wave == lead && fill) {
            if (lane >= n_fin) r.lo = sh.surv[lane];
            if (lane + WAVE >= n_fin) r.hi = sh.surv[lane + WAVE];
        }
    } else {
        exact();
    }
    finish();
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
    tile_process<DT>(P, row, tile, in, sh, to_regs);
}

}  // namespace ssd
