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
// those past the end of V take the smallest pattern.  Each lane takes the
// maximum of every 16-byte chunk and of its whole slice; each wave finds the
// k-th largest of its 64 lane maxima, k = 32 + ceil(L/4) for L listed
// tokens in the tile, and the smallest of the four is a threshold tau with
// at least 128 + L tokens at or above it - so the 128 best unlisted tokens
// are all at or above tau.  Chunks whose maximum reaches tau (typically a
// few dozen per wave) are copied from registers to the wave's LDS area;
// each lane then takes one such chunk, and the elements >= tau that are not
// listed become keys.  Each wave sorts its keys in registers, and a
// two-level merge tree gives the tile's 128.  Tiles where the test does not
// apply (tau <= 0, a positive NaN, more listed tokens or survivors than the
// LDS areas hold) take the general path: exact keys for every element and a
// bisection for the 128th key.
#pragma once

#include "ss_device.h"
#include "ss_wavesort.h"

namespace ssd {

typedef short s16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ s16x2 bits_s16x2(uint32_t u) { return __builtin_bit_cast(s16x2, u); }
__device__ __forceinline__ uint32_t s16x2_bits(s16x2 v) { return __builtin_bit_cast(uint32_t, v); }

constexpr int S1_THREADS = 256;
constexpr int S1_WAVES = S1_THREADS / WAVE;
constexpr int S1_CCAP = 128;          // flagged chunks held per wave (fast path)
constexpr int S1_KCAP = 256;          // survivors held per wave (fast path)
constexpr int S1_LIST_CAP = 512;      // >= 255 prior + 255 bias entries
constexpr int S1_NL_FAST = 128;       // listed tokens per tile the fast path absorbs

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
    using Key = typename S1Traits<DT>::Key;
    uint4 chunks[S1_WAVES][S1_CCAP];   // flagged 16-byte chunks, per wave (fast path)
    int cid[S1_WAVES][S1_CCAP];        // their chunk index in the tile
    Key keys[S1_WAVES][S1_KCAP];       // survivors per wave (fast path); general path: flat
    Key wl[S1_WAVES][KMAX];            // per-wave sorted lists
    Key surv[KMAX];                    // result: the tile's 128 best, sorted
    int listed[S1_LIST_CAP];           // tile-local indices of listed tokens
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

// Bitonic sort (descending) of 64 keys, one per lane.
template <int KS, int J, typename K>
__device__ __forceinline__ void sort64_substeps(K& v) {
    const int lane = lane_id();
    const bool keep_max = ((lane & J) == 0) == ((lane & KS) == 0);
    const K p = xor_key<J>(v);
    v = keep_max ? kmax(v, p) : kmin(v, p);
    if constexpr (J > 1) sort64_substeps<KS, J / 2>(v);
}
template <int KS = 2, typename K>
__device__ __forceinline__ void wave_sort64(K& v) {
    sort64_substeps<KS, KS / 2>(v);
    if constexpr (KS < 64) wave_sort64<KS * 2>(v);
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

// The 128 best tokens of tile `tile` of row `row`, sorted best first, left
// in sh.surv[0..128) (key 0 = no token).  Ends with a barrier.
template <int DT>
__device__ __forceinline__ void stage1_tile(const Stage1Params& P, int row, int tile, S1Shared<DT>& sh) {
    using T = S1Traits<DT>;
    using Key = typename T::Key;
    constexpr int EPC = T::EPC;
    constexpr int BN = T::BN;
    constexpr int CPT = BN / (EPC * S1_THREADS);   // 16-byte chunks per thread
    constexpr int NQ = CPT * 4;                    // dwords per thread
    static_assert(CPT * EPC <= 64, "per-thread masks hold 64 bits");
    static_assert(S1_WAVES == 4, "merge tree");
    // smallest pattern when read as signed 16-bit halves / 32-bit word: the
    // value given to grammar-masked elements and to those past the end of V
    constexpr uint32_t PAD = DT == SS_BF16 ? 0x80008000u : 0x80000000u;

    const int tid = threadIdx.x;
    const int wave = tid / WAVE;
    const int lane = lane_id();
    const uint64_t lt = (1ull << lane) - 1ull;
    const int base = tile * BN;
    const int nvalid = min(BN, P.V - base);
    const int b = row / P.rows_per_req;

    // ---- issue the tile's loads: chunk j of thread t is tile chunk j*256 + t
    // (each wave instruction reads 1 KiB of consecutive bytes) ----
    const bool full = (nvalid == BN);
    const bool vec = full && P.aligned16;
    const char* rowp = (const char*)P.logits + ((int64_t)row * P.ld + base) * (DT == SS_BF16 ? 2 : 4);
    // dword q of thread tid = dword (q & 3) of chunk (q >> 2); elements past
    // the end of V read as PAD
    auto load_dword = [&](int q) -> uint32_t {
        const int c = (q >> 2) * S1_THREADS + tid;
        if (vec) return gmem((const uint32_t*)rowp)[c * 4 + (q & 3)];
        if (DT == SS_BF16) {
            const auto p16 = gmem((const uint16_t*)rowp);
            const int e0 = c * EPC + 2 * (q & 3);
            const uint32_t lo = e0 < nvalid ? p16[e0] : 0x8000u;
            const uint32_t hi = e0 + 1 < nvalid ? p16[e0 + 1] : 0x8000u;
            return lo | (hi << 16);
        } else {
            const int e = c * EPC + (q & 3);
            return e < nvalid ? gmem((const uint32_t*)rowp)[e] : PAD;
        }
    };
    uint32_t raw[NQ];
    if (vec) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const vu32x4 v = gmem((const vu32x4*)rowp)[j * S1_THREADS + tid];
            raw[4 * j + 0] = v.x;
            raw[4 * j + 1] = v.y;
            raw[4 * j + 2] = v.z;
            raw[4 * j + 3] = v.w;
        }
    } else {
        // ragged or unaligned tile: whole chunks still load as 16 bytes
        // where they can
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int c = j * S1_THREADS + tid;
            if (P.aligned16 && (c + 1) * EPC <= nvalid) {
                const vu32x4 v = gmem((const vu32x4*)rowp)[c];
                raw[4 * j + 0] = v.x;
                raw[4 * j + 1] = v.y;
                raw[4 * j + 2] = v.z;
                raw[4 * j + 3] = v.w;
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) raw[4 * j + k] = load_dword(4 * j + k);
            }
        }
    }

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

    // grammar bits of each chunk (bit e: element e allowed); one byte of
    // the row's bitmask covers 8 tokens
    uint32_t gbits[CPT];
    if (use_grammar) {
        const auto gm = gmem((const uint8_t*)(P.aux.bitmask + (int64_t)row * P.aux.bitmask_stride));
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const int g0 = base + (j * S1_THREADS + tid) * EPC;
            uint32_t g = g0 < P.V ? (uint32_t)gm[g0 >> 3] : 0u;
            if (DT == SS_F32) g >>= (g0 & 4);
            gbits[j] = g;
        }
    }

    // ---- tokens of this tile named by an active list: ranked in Stage 2,
    // left out here.  Every wave counts them; wave 0 also records them. ----
    int nl = 0;
    if (use_prior) {
        const auto ids = gmem(P.aux.prior_ids + (int64_t)b * P.aux.prior_stride);
        const auto cts = gmem(P.aux.prior_cnt + (int64_t)b * P.aux.prior_stride);
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
            if (wave == 0 && ok) sh.listed[nl + __popcll(bal & lt)] = loc;
            nl += __popcll(bal);
        }
    }
    if (use_bias) {
        const auto ids = gmem(P.aux.bias_ids + (int64_t)b * P.aux.bias_stride);
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
            if (wave == 0 && ok) sh.listed[nl + __popcll(bal & lt)] = loc;
            nl += __popcll(bal);
        }
    }
    if (tid == 0) sh.ovf = 0;

    // ---- grammar: masked elements take PAD ----
    if (use_grammar) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const uint32_t g = gbits[j];
            if (DT == SS_BF16) {
                // bit 2k -> low half of dword k, bit 2k+1 -> high half
                const s16x2 G = bits_s16x2(g | (g << 16));
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const s16x2 sh_l = {(short)(15 - 2 * k), (short)(14 - 2 * k)};
                    const s16x2 sh_r = {15, 15};
                    const uint32_t M = s16x2_bits((G << sh_l) >> sh_r);
                    raw[4 * j + k] = (raw[4 * j + k] & M) | (PAD & ~M);
                }
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t M = 0u - ((g >> k) & 1u);
                    raw[4 * j + k] = (raw[4 * j + k] & M) | (PAD & ~M);
                }
            }
        }
    }

    // ---- maxima per chunk and per lane (raw patterns read as signed) ----
    uint32_t cmx[CPT];
    int m;
    if constexpr (DT == SS_BF16) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const s16x2 a = __builtin_elementwise_max(bits_s16x2(raw[4 * j]), bits_s16x2(raw[4 * j + 1]));
            const s16x2 c = __builtin_elementwise_max(bits_s16x2(raw[4 * j + 2]), bits_s16x2(raw[4 * j + 3]));
            cmx[j] = s16x2_bits(__builtin_elementwise_max(a, c));
        }
        s16x2 mm = bits_s16x2(cmx[0]);
#pragma unroll
        for (int j = 1; j < CPT; ++j) mm = __builtin_elementwise_max(mm, bits_s16x2(cmx[j]));
        m = max((int)mm.x, (int)mm.y);
    } else {
#pragma unroll
        for (int j = 0; j < CPT; ++j)
            cmx[j] = (uint32_t)max(max((int)raw[4 * j], (int)raw[4 * j + 1]),
                                   max((int)raw[4 * j + 2], (int)raw[4 * j + 3]));
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
    const bool nl_ok = nl <= S1_NL_FAST;
    const int kw = KMAX / S1_WAVES + (nl_ok ? (nl + S1_WAVES - 1) / S1_WAVES : 0);
    const int tau_w = wave_kth_largest<T::VAL_BITS>(m, kw);
    const uint64_t sp = __ballot(special);
    if (lane == 0) {
        sh.tau[wave] = tau_w;
        sh.special[wave] = sp != 0ull;
    }
    __syncthreads();   // tau, listed[], ovf
    int tau = sh.tau[0];
    bool any_special = false;
#pragma unroll
    for (int w = 0; w < S1_WAVES; ++w) {
        tau = min(tau, sh.tau[w]);
        any_special |= sh.special[w] != 0;
    }
    const bool fast = !any_special && tau >= 1 && nl_ok;   // block-uniform

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
            if (f) {
                const int s = wcnt + __popcll(bal & lt);
                if (s < S1_CCAP) {
                    sh.chunks[wave][s] = make_uint4(raw[4 * j], raw[4 * j + 1], raw[4 * j + 2], raw[4 * j + 3]);
                    sh.cid[wave][s] = j * S1_THREADS + tid;
                }
            }
            wcnt += __popcll(bal);
        }
        wave_lds_sync();

        // ---- the survivors of those chunks become keys (listed ones dropped) ----
        const int nck = min(wcnt, S1_CCAP);
        int nk = 0;
        for (int s0 = 0; s0 < nck; s0 += WAVE) {
            const int s = s0 + lane;
            uint4 d = make_uint4(PAD, PAD, PAD, PAD);
            int c = -1;
            if (s < nck) {
                d = sh.chunks[wave][s];
                c = sh.cid[wave][s];
            }
            uint32_t ex = 0;
            for (int i = 0; i < nl; ++i) {
                const int loc = sh.listed[i];
                if (loc / EPC == c) ex |= 1u << (loc % EPC);
            }
            const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                uint32_t h;
                int v;
                if constexpr (DT == SS_BF16) {
                    h = (dw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                    v = (int)(short)h;
                } else {
                    h = dw[e];
                    v = (int)h;
                }
                const bool sv = v >= tau && !((ex >> e) & 1u);
                const uint64_t bal = __ballot(sv);
                if (sv) {
                    const int slot = nk + __popcll(bal & lt);
                    const int local = c * EPC + e;
                    if (slot < S1_KCAP) {
                        // value > 0 and not NaN here
                        if constexpr (DT == SS_BF16)
                            sh.keys[wave][slot] = ((h | 0x8000u) << 16) | (0xFFFFu - (uint32_t)local);
                        else
                            sh.keys[wave][slot] = key_f32(h, local, true, true);
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
    }
    __syncthreads();   // wave lists, ovf

    if (fast && sh.ovf == 0) {
        // ---- merge tree: (0+1) on wave 0 and (2+3) on wave 1, then both ----
        WList<Key> r{0, 0};
        if (wave < 2) {
            const int a = 2 * wave;
            r = wave_merge(WList<Key>{sh.wl[a][lane], sh.wl[a][lane + WAVE]},
                           WList<Key>{sh.wl[a + 1][lane], sh.wl[a + 1][lane + WAVE]});
            if (wave == 1) {
                sh.wl[2][lane] = r.lo;
                sh.wl[2][lane + WAVE] = r.hi;
            }
        }
        __syncthreads();
        if (wave == 0) {
            r = wave_merge(r, WList<Key>{sh.wl[2][lane], sh.wl[2][lane + WAVE]});
            sh.surv[lane] = r.lo;
            sh.surv[lane + WAVE] = r.hi;
        }
        __syncthreads();
        return;
    }

    // ---- general path: exact keys for every element (re-read from cache),
    // bisection for the 128th key ----
    const uint32_t all_bits = (1u << EPC) - 1u;
    uint64_t alw = ~0ull, pres = ~0ull, excl = 0;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const int c0 = (j * S1_THREADS + tid) * EPC;
        uint32_t pb = all_bits;
        if (!full) pb = c0 >= nvalid ? 0u : (nvalid - c0 >= EPC ? all_bits : ((1u << (nvalid - c0)) - 1u));
        pres &= ~((uint64_t)(all_bits & ~pb) << (j * EPC));
        if (use_grammar && pb) {
            const int g0 = base + c0;
            const uint32_t w = gmem(P.aux.bitmask)[(int64_t)row * P.aux.bitmask_stride + (g0 >> 5)];
            alw &= ~((uint64_t)(all_bits & ~((w >> (g0 & 31)) & all_bits)) << (j * EPC));
        }
    }
    for (int i = 0; i < nl; ++i) {
        const int loc = sh.listed[i];
        const int c = loc / EPC;
        if ((c & (S1_THREADS - 1)) == tid) excl |= 1ull << ((c / S1_THREADS) * EPC + (loc % EPC));
    }
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
    int off = block_excl_scan(cnt, sh.scan, &total);   // total <= 128 (keys are unique)
    Key* g = &sh.keys[0][0];
    for (int q = 0; q < NQ; ++q)
        for (int h = 0; h < HALVES; ++h) {
            const Key k = ekey(q, h);
            if (k >= thr) g[off++] = k;
        }
    __syncthreads();
    if (wave == 0) {
        WList<Key> l{lane < total ? g[lane] : (Key)0, lane + WAVE < total ? g[lane + WAVE] : (Key)0};
        l = wave_sort128(l);
        sh.surv[lane] = l.lo;
        sh.surv[lane + WAVE] = l.hi;
    }
    __syncthreads();
}

}  // namespace ssd
