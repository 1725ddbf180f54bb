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
// Selection is exact.  Fast path: each lane takes the maximum of its
// elements; each wave finds the 32nd largest of its 64 lane maxima; the
// smallest of the four is a threshold tau with at least 128 tokens at or
// above it, so the tile's 128 best are among the survivors x >= tau
// (typically ~200 of 16384).  On raw bit patterns read as signed integers
// the comparison x >= tau agrees with the float order whenever tau > 0, so
// the fast path needs no per-element key transform.  Tiles where the test
// does not apply (tau <= 0, a positive NaN, too many survivors) take the
// general path: exact keys for every element and a bisection for the 128th
// key.  Both paths end in bitonic sorts of the survivors held in registers
// (one 128-key chunk per wave) and a merge of the per-wave lists.
#pragma once

#include "ss_device.h"
#include "ss_wavesort.h"

namespace ssd {

typedef short s16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ s16x2 bits_s16x2(uint32_t u) { return __builtin_bit_cast(s16x2, u); }
__device__ __forceinline__ uint32_t s16x2_bits(s16x2 v) { return __builtin_bit_cast(uint32_t, v); }

constexpr int S1_THREADS = 256;
constexpr int S1_WAVES = S1_THREADS / WAVE;
constexpr int S1_SURV_CAP = 1024;     // survivors held in LDS (fast path)
constexpr int S1_LIST_CAP = 512;      // >= 255 prior + 255 bias entries

template <int DT> struct S1Traits;
template <> struct S1Traits<SS_BF16> {
    using Key = uint32_t;
    static constexpr int EPC = 8;          // elements per 16-byte chunk
    static constexpr int BN = 16384;       // tile width
    static constexpr int VAL_BITS = 16;    // fast-path value range (int16)
};
template <> struct S1Traits<SS_F32> {
    using Key = uint64_t;
    static constexpr int EPC = 4;
    static constexpr int BN = 8192;
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
    int listed_rows;     // workgroups 0 .. listed_rows-1 compute them
    int aligned16;       // rows start on 16-byte boundaries
};

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
    typename S1Traits<DT>::Key surv[S1_SURV_CAP];
    typename S1Traits<DT>::Key wl[S1_WAVES][KMAX];
    int listed[S1_LIST_CAP];
    int nlisted;
    int tau[S1_WAVES];
    int special[S1_WAVES];
    int scan[S1_WAVES];
    int red[2][S1_WAVES];
};

// The 128 best tokens of tile `tile` of row `row`, sorted best first, left
// in sh.surv[0..128) (key 0 = no token).  Ends with a barrier.
template <int DT>
__device__ void stage1_tile(const Stage1Params& P, int row, int tile, S1Shared<DT>& sh) {
    using T = S1Traits<DT>;
    using Key = typename T::Key;
    constexpr int EPC = T::EPC;
    constexpr int BN = T::BN;
    constexpr int CPT = BN / (EPC * S1_THREADS);   // 16-byte chunks per thread
    static_assert(CPT * EPC <= 64, "per-thread exclusion mask holds 64 bits");
    Key* surv = sh.surv;
    int* listed = sh.listed;

    const int tid = threadIdx.x;
    const int wave = tid / WAVE;
    const int lane = lane_id();
    const int base = tile * BN;
    const int nvalid = min(BN, P.V - base);
    const int b = row / P.rows_per_req;

    uint32_t flags = 0;
    int n_prior = 0, n_bias = 0;
    if (P.req) {
        const ss_req r = P.req[b];
        flags = r.flags;
        // a list longer than its stride makes the row invalid (reported by
        // Stage 2); the tiles then use no list at all
        n_prior = (int)r.n_prior <= P.aux.prior_stride ? (int)r.n_prior : 0;
        n_bias = (int)r.n_bias <= P.aux.bias_stride ? (int)r.n_bias : 0;
    }
    const bool use_grammar = (flags & SS_GRAMMAR) && P.aux.bitmask;
    const bool use_prior = (flags & (SS_REP | SS_FREQPRES)) && P.aux.prior_ids && P.aux.prior_cnt && n_prior > 0;
    const bool use_bias = (flags & SS_BIAS) && P.aux.bias_ids && n_bias > 0;

    // ---- tokens of this tile named by an active list (left out here) ----
    if (wave == 0) {
        int cnt = 0;
        const uint64_t lt = (1ull << lane) - 1ull;
        if (use_prior) {
            const int32_t* ids = P.aux.prior_ids + (int64_t)b * P.aux.prior_stride;
            const int32_t* cts = P.aux.prior_cnt + (int64_t)b * P.aux.prior_stride;
            for (int j0 = 0; j0 < n_prior; j0 += WAVE) {
                const int j = j0 + lane;
                bool ok = false;
                int loc = 0;
                if (j < n_prior) {
                    const int id = ids[j];
                    loc = id - base;
                    ok = cts[j] >= 1 && id >= 0 && id < P.V && loc >= 0 && loc < nvalid;
                }
                const uint64_t bal = __ballot(ok);
                if (ok) listed[cnt + __popcll(bal & lt)] = loc;
                cnt += __popcll(bal);
            }
        }
        if (use_bias) {
            const int32_t* ids = P.aux.bias_ids + (int64_t)b * P.aux.bias_stride;
            for (int j0 = 0; j0 < n_bias; j0 += WAVE) {
                const int j = j0 + lane;
                bool ok = false;
                int loc = 0;
                if (j < n_bias) {
                    const int id = ids[j];
                    loc = id - base;
                    ok = id >= 0 && id < P.V && loc >= 0 && loc < nvalid;
                }
                const uint64_t bal = __ballot(ok);
                if (ok) listed[cnt + __popcll(bal & lt)] = loc;
                cnt += __popcll(bal);
            }
        }
        if (lane == 0) sh.nlisted = cnt;
    }

    // ---- load the tile: chunk j of thread t is tile chunk j*256 + t ----
    // (each wave instruction reads 1 KiB of consecutive bytes)
    const bool full = (nvalid == BN);
    const char* rowp = (const char*)P.logits + ((int64_t)row * P.ld + base) * (DT == SS_BF16 ? 2 : 4);
    // dword q of thread tid = dword (q & 3) of chunk (q >> 2)
    auto load_dword = [&](int q) -> uint32_t {
        const int c = (q >> 2) * S1_THREADS + tid;
        if (full && P.aligned16) return ((const uint32_t*)rowp)[c * 4 + (q & 3)];
        if (DT == SS_BF16) {
            const uint16_t* p16 = (const uint16_t*)rowp;
            const int e0 = c * EPC + 2 * (q & 3);
            const uint32_t lo = e0 < nvalid ? p16[e0] : 0u;
            const uint32_t hi = e0 + 1 < nvalid ? p16[e0 + 1] : 0u;
            return lo | (hi << 16);
        } else {
            const int e = c * EPC + (q & 3);
            return e < nvalid ? ((const uint32_t*)rowp)[e] : 0u;
        }
    };
    constexpr int NQ = CPT * 4;   // dwords per thread
    uint32_t raw[NQ];
    if (full && P.aligned16) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const uint4 v = *((const uint4*)rowp + (j * S1_THREADS + tid));
            raw[4 * j + 0] = v.x;
            raw[4 * j + 1] = v.y;
            raw[4 * j + 2] = v.z;
            raw[4 * j + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int q = 0; q < NQ; ++q) raw[q] = load_dword(q);
    }

    // ---- per-element bits: present (inside V), allowed by the grammar, not listed ----
    // element e of chunk j is bit j*EPC + e
    const uint32_t all_bits = (1u << EPC) - 1u;
    uint64_t alw = ~0ull, pres = ~0ull;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c0 = (j * S1_THREADS + tid) * EPC;
        uint32_t pb = all_bits;
        if (!full) pb = c0 >= nvalid ? 0u : (nvalid - c0 >= EPC ? all_bits : ((1u << (nvalid - c0)) - 1u));
        pres &= ~((uint64_t)(all_bits & ~pb) << (j * EPC));
        if (use_grammar && pb) {
            const int g0 = base + c0;
            const uint32_t w = P.aux.bitmask[(int64_t)row * P.aux.bitmask_stride + (g0 >> 5)];
            alw &= ~((uint64_t)(all_bits & ~((w >> (g0 & 31)) & all_bits)) << (j * EPC));
        }
    }
    __syncthreads();   // listed[] ready
    const int nlisted = sh.nlisted;
    uint64_t excl = 0;
    for (int i = 0; i < nlisted; ++i) {
        const int loc = listed[i];
        const int c = loc / EPC;
        if ((c & (S1_THREADS - 1)) == tid) excl |= 1ull << ((c / S1_THREADS) * EPC + (loc % EPC));
    }
    const uint64_t inc = alw & pres & ~excl;
    const bool need_mask = !full || use_grammar || nlisted > 0;   // block-uniform

    // ---- fast-path values: raw patterns as signed integers; left-out -> minimum ----
    if (need_mask) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if (DT == SS_BF16) {
                const uint32_t b2 = (uint32_t)(inc >> (2 * q)) & 3u;
                const uint32_t M = ((b2 & 1u) ? 0x0000FFFFu : 0u) | ((b2 & 2u) ? 0xFFFF0000u : 0u);
                raw[q] = (raw[q] & M) | (0x80008000u & ~M);
            } else {
                if (!((inc >> q) & 1ull)) raw[q] = 0x80000000u;
            }
        }
    }
    int m;
    if (DT == SS_BF16) {
        s16x2 mx = bits_s16x2(raw[0]);
#pragma unroll
        for (int q = 1; q < NQ; ++q) mx = __builtin_elementwise_max(mx, bits_s16x2(raw[q]));
        m = max((int)mx.x, (int)mx.y);
    } else {
        m = (int)raw[0];
#pragma unroll
        for (int q = 1; q < NQ; ++q) m = max(m, (int)raw[q]);
    }

    // positive NaN anywhere in the tile -> general path; +inf of fp32 counts
    // as FLT_MAX for the threshold
    const int nan_floor = DT == SS_BF16 ? 0x7F80 : (int)F32_PINF_BITS;
    const bool special = m > nan_floor;
    if (DT == SS_F32) m = min(m, (int)F32_MAX_BITS);
    const int tau_w = wave_kth_largest<T::VAL_BITS>(m, KMAX / S1_WAVES);
    const uint64_t sp = __ballot(special);
    if (lane == 0) {
        sh.tau[wave] = tau_w;
        sh.special[wave] = sp != 0ull;
    }
    __syncthreads();
    int tau = sh.tau[0];
    bool any_special = false;
#pragma unroll
    for (int w = 0; w < S1_WAVES; ++w) {
        tau = min(tau, sh.tau[w]);
        any_special |= sh.special[w] != 0;
    }

    bool fast = !any_special && tau >= 1;
    int nsurv = 0;
    if (fast) {
        // dwords holding a survivor (value >= tau)
        uint32_t smask = 0;
        if (m >= tau) {
            if (DT == SS_BF16) {
                const uint32_t T2 = ((uint32_t)(tau - 1) & 0xFFFFu) * 0x10001u;
                const s16x2 tv = bits_s16x2(T2);
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const s16x2 r = __builtin_elementwise_max(bits_s16x2(raw[q]), tv);
                    smask |= (s16x2_bits(r) != T2) ? (1u << q) : 0u;
                }
            } else {
#pragma unroll
                for (int q = 0; q < NQ; ++q) smask |= ((int)raw[q] >= tau) ? (1u << q) : 0u;
            }
        }
        // survivors per thread (re-reading the few dwords from cache)
        auto survivor_bits = [&](int q, uint32_t d) -> uint32_t {
            if (DT == SS_BF16) {
                const uint32_t b2 = (uint32_t)(inc >> (2 * q)) & 3u;
                uint32_t r = 0;
                if ((b2 & 1u) && (int)(short)(d & 0xFFFFu) >= tau) r |= 1u;
                if ((b2 & 2u) && ((int)d >> 16) >= tau) r |= 2u;
                return r;
            } else {
                return ((inc >> q) & 1ull) && (int)d >= tau ? 1u : 0u;
            }
        };
        int cnt = 0;
        for (uint32_t sm = smask; sm; sm &= sm - 1) {
            const int q = __builtin_ctz(sm);
            cnt += __builtin_popcount(survivor_bits(q, load_dword(q)));
        }
        int total;
        int off = block_excl_scan(cnt, sh.scan, &total);
        if (total <= S1_SURV_CAP) {
            nsurv = total;
            for (uint32_t sm = smask; sm; sm &= sm - 1) {
                const int q = __builtin_ctz(sm);
                const uint32_t d = load_dword(q);
                const uint32_t sb = survivor_bits(q, d);
                const int c = (q >> 2) * S1_THREADS + tid;
                if (DT == SS_BF16) {
                    const int e0 = c * EPC + 2 * (q & 3);
                    if (sb & 1u) surv[off++] = (Key)key_bf16(d & 0xFFFFu, e0, true, true);
                    if (sb & 2u) surv[off++] = (Key)key_bf16(d >> 16, e0 + 1, true, true);
                } else {
                    if (sb) surv[off++] = (Key)key_f32(d, c * EPC + (q & 3), true, true);
                }
            }
        } else {
            fast = false;   // block-uniform: total is the same everywhere
        }
    }

    if (!fast) {
        // ---- general path: exact keys (re-read from cache), bisection for the 128th key ----
        auto ekey = [&](int q, int h) -> Key {
            const uint32_t d = load_dword(q);
            const int c = (q >> 2) * S1_THREADS + tid;
            if (DT == SS_BF16) {
                const int e = 2 * (q & 3) + h;
                const int bitpos = (q >> 2) * EPC + e;
                const bool present = ((pres & ~excl) >> bitpos) & 1ull;
                const bool allowed = (alw >> bitpos) & 1ull;
                return (Key)key_bf16(h ? (d >> 16) : (d & 0xFFFFu), c * EPC + e, present, allowed);
            } else {
                const int bitpos = q;
                const bool present = ((pres & ~excl) >> bitpos) & 1ull;
                const bool allowed = (alw >> bitpos) & 1ull;
                return (Key)key_f32(d, c * EPC + (q & 3), present, allowed);
            }
        };
        constexpr int HALVES = DT == SS_BF16 ? 2 : 1;
        constexpr int KB = (int)sizeof(Key) * 8;
        Key res = 0;
        int parity = 0;
        for (int bit = KB - 1; bit >= 0; --bit) {
            const Key cand = res | ((Key)1 << bit);
            int c = 0;
            for (int q = 0; q < NQ; ++q)
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
        for (int q = 0; q < NQ; ++q)
            for (int h = 0; h < HALVES; ++h) cnt += ekey(q, h) >= thr;
        int total;
        int off = block_excl_scan(cnt, sh.scan, &total);
        nsurv = total;   // <= 128 (keys are unique)
        for (int q = 0; q < NQ; ++q)
            for (int h = 0; h < HALVES; ++h) {
                const Key k = ekey(q, h);
                if (k >= thr) surv[off++] = k;
            }
    }

    // ---- the 128 best survivors, sorted: each wave sorts 128-key chunks in
    // registers and keeps the best 128 of its chunks; wave 0 merges the
    // per-wave lists (key 0 = no token) ----
    __syncthreads();   // survivors complete
    const int nchunks = (nsurv + KMAX - 1) / KMAX;
    WList<Key> mine{0, 0};
    for (int c = wave; c < nchunks; c += S1_WAVES) {
        const int i0 = c * KMAX + lane, i1 = i0 + WAVE;
        WList<Key> l{i0 < nsurv ? surv[i0] : (Key)0, i1 < nsurv ? surv[i1] : (Key)0};
        l = wave_sort128(l);
        mine = c == wave ? l : wave_merge(mine, l);
    }
    if (nchunks > 1) {
        sh.wl[wave][lane] = mine.lo;
        sh.wl[wave][lane + WAVE] = mine.hi;
        __syncthreads();
        if (wave == 0)
            for (int w = 1; w < S1_WAVES && w < nchunks; ++w)
                mine = wave_merge(mine, WList<Key>{sh.wl[w][lane], sh.wl[w][lane + WAVE]});
    }
    if (wave == 0) {
        surv[lane] = mine.lo;
        surv[lane + WAVE] = mine.hi;
    }
    __syncthreads();
}

}  // namespace ssd
