// Stage-1 tile selection by the adaptive radix-bitonic strategy of the
// SonicSampler paper (Fig. 1, right panel: a reduction tree screens the 6
// most significant bits of the order key, then either a radix select over
// the low 10 bits runs or the bitonic select finishes at once), for plain
// top-k (no logits processing), as the alternative to the threshold select of
// ss_stage1.h.
//
// Per tile workgroup:
//   * the 16-bit screening key of an element is its bf16 order key, or the
//     upper half of its fp32 order key;
//   * screen: every thread counts its elements' top-6-bit buckets in its own
//     LDS column (no two threads touch one word, and a wave's 64 columns lie
//     on distinct banks, so the increments neither contend nor conflict),
//     and a reduction tree sums the columns into 64 bucket totals; the
//     bucket holding the 128th best element follows from a scan;
//   * if the elements at or above that bucket number at most 256 they go
//     to the bitonic select directly; otherwise one radix pass counts the
//     low 10 bits of the bucket's elements in a shared 1024-entry histogram
//     and a block scan gives the 16-bit key of the 128th best;
//   * the elements at or above the bucket or key found are compacted as
//     exact keys (value, then lower id first) and the wave bitonic network
//     keeps the best 128;
//   * more than 256 elements tied at 16-bit precision take the exact
//     threshold path of ss_stage1.h instead.
// The output is the same sorted tile list as stage1_kernel's.
#pragma once

#include <type_traits>

#include "ss_stage1.h"

namespace ssd {

constexpr int RX_CAP = 256;            // exact keys the bitonic finish takes
constexpr int RX_NB1 = 64;             // screen: the 6 most significant bits
constexpr int RX_NB2 = 1024;           // refinement: the next 10 bits

template <int DT>
struct RadixShared {
    using Key = typename S1Traits<DT>::Key;
    alignas(16) uint32_t col[RX_NB1][S1_THREADS];  // screen: thread t's count of bucket b at [b][t]
    alignas(16) uint32_t hist[RX_NB2 + WAVE];      // refinement counts; entry RX_NB2 + lane takes a lane's elements out of range
    uint32_t h1[RX_NB1];               // screen bucket totals
    Key keys[RX_CAP + WAVE];           // candidates; the last WAVE entries take the other lanes' writes
    int wsum[S1_WAVES];
    int flag[S1_WAVES];
    int sel[3];   // bucket of the 128th best (-1: fewer elements than needed), count above it, its count
};

template <int DT>
union RadixKernelShared {
    S1Shared<DT> tile;
    RadixShared<DT> rad;
};

// The heavy-tie case: the threshold path reloads the tile itself, so none
// of the caller's key registers live across it.
template <int DT>
__device__ __forceinline__ void radix_tie_fallback(const Stage1Params& P, int row, int tile, S1Shared<DT>& st) {
    using Key = typename S1Traits<DT>::Key;
    WList<Key> res{0, 0};
    stage1_tile<DT>(P, row, tile, st, &res);
    if ((int)threadIdx.x / WAVE == s1_lead_wave()) {
        const int64_t o = ((int64_t)row * P.Zv + tile) * KMAX + lane_id();
        ((Key*)P.scratch)[o] = res.lo;
        ((Key*)P.scratch)[o + WAVE] = res.hi;
    }
}

using u16x2 = unsigned short __attribute__((ext_vector_type(2)));

// The fast screen of stage1_radix_kernel (see there): true when it has
// written the tile's list.  Block-uniform result; kk holds the tile's order
// keys (bf16: two 16-bit keys per dword; fp32: one 32-bit key), 0 past the
// end.
template <int DT>
__device__ __forceinline__ bool rx_fast_screen(const Stage1Params& P, int row, int tile, const uint32_t (&kk)[S1_CPT * 4],
                                               RadixShared<DT>& sh, int nvalid) {
    using Key = typename S1Traits<DT>::Key;
    constexpr int EPC = S1Traits<DT>::EPC;
    constexpr int BN = S1Traits<DT>::BN;
    constexpr int NCH = S1_CPT;
    const int tid = threadIdx.x, wave = tid / WAVE, lane = lane_id();
    // this thread's chunk maxima (screening keys); chunk j is tile chunk j * 256 + tid
    uint32_t cmx[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        if constexpr (DT == SS_BF16) {
            u16x2 m = __builtin_bit_cast(u16x2, kk[4 * j]);
#pragma unroll
            for (int i = 1; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, kk[4 * j + i]));
            cmx[j] = m[0] > m[1] ? m[0] : m[1];
        } else {
            const uint32_t a = kk[4 * j] > kk[4 * j + 1] ? kk[4 * j] : kk[4 * j + 1];
            const uint32_t c = kk[4 * j + 2] > kk[4 * j + 3] ? kk[4 * j + 2] : kk[4 * j + 3];
            cmx[j] = (a > c ? a : c) >> 16;
        }
    }
    const int nzc = BN / EPC - (nvalid + EPC - 1) / EPC;   // chunks with no element: maximum 0
    if (BN / EPC - nzc < KMAX) return false;               // block-uniform
    // 6-bit screen of the chunk maxima, per-thread LDS columns as below
#pragma unroll
    for (int b = 0; b < RX_NB1; ++b) sh.col[b][tid] = 0u;
#pragma unroll
    for (int i = tid; i < RX_NB2; i += S1_THREADS) sh.hist[i] = 0u;
#pragma unroll
    for (int j = 0; j < NCH; ++j)
        __hip_atomic_fetch_add(&sh.col[cmx[j] >> 10][tid], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __syncthreads();
    {
        const int b = tid >> 2, part = tid & 3;
        const uint4* src = (const uint4*)&sh.col[b][part * 64];
        uint32_t s = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint4 v = src[(i + b) & 15];
            s += v.x + v.y + v.z + v.w;
        }
        s += xor_lane<1>(s);
        s += xor_lane<2>(s);
        if (part == 0) sh.h1[b] = s;
    }
    __syncthreads();
    if (wave == 0) {
        int c = (int)sh.h1[RX_NB1 - 1 - lane];
        if (lane == RX_NB1 - 1) c -= nzc;
        const int incl = wave_incl_scan(c);
        const uint64_t reach = __ballot(incl >= KMAX);
        const int l = reach ? __builtin_ctzll(reach) : 0;
        if (lane == 0) {
            sh.sel[0] = RX_NB1 - 1 - l;
            sh.sel[1] = __builtin_amdgcn_readlane(incl, l) - __builtin_amdgcn_readlane(c, l);
        }
    }
    __syncthreads();
    // 10-bit refinement inside that bucket: T0 exactly
    const int d = sh.sel[0];
    const int need = KMAX - sh.sel[1];
    const uint32_t lo = (uint32_t)d << 10;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const uint32_t dg = cmx[j] - lo;
        if (dg < (uint32_t)RX_NB2)
            __hip_atomic_fetch_add(&sh.hist[dg], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
    {
        const uint4 v = *(const uint4*)&sh.hist[RX_NB2 - 4 - 4 * tid];
        uint32_t c3 = v.w, c2 = v.z, c1 = v.y, c0 = v.x;
        if (tid == S1_THREADS - 1 && d == 0) c0 -= nzc;
        const int s = (int)(c0 + c1 + c2 + c3);
        const int wincl = wave_incl_scan(s);
        if (lane == WAVE - 1) sh.wsum[wave] = wincl;
        __syncthreads();
        int before = wincl - s;
#pragma unroll
        for (int w = 0; w < S1_WAVES; ++w) before += w < wave ? sh.wsum[w] : 0;
        const int cs[4] = {(int)c3, (int)c2, (int)c1, (int)c0};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (before < need && before + cs[j] >= need) sh.sel[2] = RX_NB2 - 1 - 4 * tid - j;   // exactly one
            before += cs[j];
        }
    }
    __syncthreads();
    const uint32_t T0 = lo + (uint32_t)sh.sel[2];   // >= 1: the 128 maxima are elements
    // the chunks whose maximum reaches T0, copied per wave (the column area
    // is free now); more than S1_CCAP in a wave takes the element screen
    uint4* const ch = (uint4*)&sh.col[0][0] + wave * (S1_CCAP + WAVE);
    int* const cid = (int*)((uint4*)&sh.col[0][0] + S1_WAVES * (S1_CCAP + WAVE)) + wave * (S1_CCAP + WAVE);
    int wcnt = 0;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const bool f = cmx[j] >= T0;
        const uint64_t bal = __ballot(f);
        if (f && wcnt <= S1_CCAP) {
            const int sl = wcnt + lane_prefix(bal);
            ch[sl] = make_uint4(kk[4 * j], kk[4 * j + 1], kk[4 * j + 2], kk[4 * j + 3]);
            cid[sl] = j * S1_THREADS + tid;
        }
        wcnt += __popcll(bal);
    }
    // the elements >= T0 of those chunks: count, then place
    const int nck = wcnt < S1_CCAP ? wcnt : S1_CCAP;
    wave_lds_sync();
    int mine = 0;
    for (int s0 = 0; s0 < nck; s0 += WAVE) {
        const int sl = s0 + lane;
        if (sl < nck) {
            const uint4 v = ch[sl];
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (DT == SS_BF16) mine += ((w4[e] & 0xFFFFu) >= T0) + ((w4[e] >> 16) >= T0);
                else mine += (w4[e] >> 16) >= T0;
            }
        }
    }
    int wtot = mine;
    wtot += xor_lane<1>(wtot);
    wtot += xor_lane<2>(wtot);
    wtot += xor_lane<4>(wtot);
    wtot += xor_lane<8>(wtot);
    wtot += xor_lane<16>(wtot);
    wtot += xor_lane<32>(wtot);
    if (lane == 0) sh.flag[wave] = wcnt > S1_CCAP ? -1 : wtot;
    __syncthreads();
    int total = 0, pos = 0;
    bool bad = false;
#pragma unroll
    for (int w = 0; w < S1_WAVES; ++w) {
        const int f = sh.flag[w];
        bad |= f < 0;
        pos += w < wave ? f : 0;
        total += f;
    }
    if (bad || total > RX_CAP) return false;   // block-uniform
    pos += wave_incl_scan(mine) - mine;
    for (int s0 = 0; s0 < nck; s0 += WAVE) {
        const int sl = s0 + lane;
        if (sl < nck) {
            const uint4 v = ch[sl];
            const int c = cid[sl];
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (DT == SS_BF16) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint32_t k16 = h ? w4[e] >> 16 : w4[e] & 0xFFFFu;
                        if (k16 >= T0) {
                            const uint32_t loc = (uint32_t)(c * EPC + 2 * e + h);
                            sh.keys[pos++] = (Key)((k16 << 16) | (0xFFFFu - loc));
                        }
                    }
                } else {
                    if ((w4[e] >> 16) >= T0) {
                        const uint32_t loc = (uint32_t)(c * EPC + e);
                        sh.keys[pos++] = (Key)(((uint64_t)w4[e] << 32) | (uint64_t)(0xFFFFFFFFu - loc));
                    }
                }
            }
        }
    }
    __syncthreads();
    if (wave == 0) {
        const WList<Key> best = wave_top128(sh.keys, total);
        const int64_t o = ((int64_t)row * P.Zv + tile) * KMAX + lane;
        ((Key*)P.scratch)[o] = best.lo;
        ((Key*)P.scratch)[o + WAVE] = best.hi;
    }
    return true;
}

template <int DT>
__global__ __launch_bounds__(S1_THREADS) void stage1_radix_kernel(Stage1Params P) {
    using Key = typename S1Traits<DT>::Key;
    __shared__ RadixKernelShared<DT> shu;
    RadixShared<DT>& sh = shu.rad;
    const int wg = blockIdx.x;
    const int row = div_uniform(wg, P.Zv);
    const int tile = wg - row * P.Zv;
    S1_TILE_GEOMETRY
    S1In<DT> in;
    tile_fetch<DT>(P, row, tile, in);
    tile_patch<DT>(P, row, tile, in);
    constexpr int HALVES = DT == SS_BF16 ? 2 : 1;
    constexpr int KB = DT == SS_BF16 ? 16 : 32;   // order-key width; the screening key is its top 16 bits
    auto local_of = [&](int q, int h) {
        const int c = (q >> 2) * S1_THREADS + tid;
        return c * EPC + (DT == SS_BF16 ? 2 * (q & 3) + h : (q & 3));
    };
    uint32_t (&kk)[NQ] = in.raw;

    // ---- the data become order keys in place: bf16 two 16-bit keys per
    // dword, fp32 one 32-bit key.  Whole aligned tiles take the plain
    // order map and only check for the values the canonical order changes
    // (NaN, +inf, -0); a tile with one of them, a ragged tile and an
    // unaligned row read every element again and map it canonically, with
    // 0 (below every element's key) past the end. ----
    if (vec) {
        bool sp = false;   // this lane saw a value the canonical order changes
        if constexpr (DT == SS_BF16) {
            u16x2 mx = {0, 0}, mn = {0xFFFF, 0xFFFF}, mz = {0xFFFF, 0xFFFF};
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const uint32_t x = kk[q];
                const uint32_t m = (x >> 15) & 0x00010001u;           // sign bits of both halves
                const uint32_t k = x ^ (m * 0x7FFFu + 0x80008000u);   // 0xFFFF or 0x8000 per half
                kk[q] = k;
                const u16x2 kv = __builtin_bit_cast(u16x2, k);
                mx = __builtin_elementwise_max(mx, kv);
                mn = __builtin_elementwise_min(mn, kv);
                mz = __builtin_elementwise_min(mz, kv ^ (u16x2){0x7FFF, 0x7FFF});
            }
            // +inf or NaN at the top, NaN at the bottom, -0 (key 0x7FFF)
            sp = mx[0] >= K16_PINF || mx[1] >= K16_PINF || mn[0] < K16_NINF || mn[1] < K16_NINF ||
                 mz[0] == 0 || mz[1] == 0;
        } else {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const uint32_t x = kk[q];
                sp |= __builtin_amdgcn_class(bitsf(x), 0x223);   // NaN, -0, +inf
                kk[q] = x ^ ((uint32_t)((int32_t)x >> 31) | 0x80000000u);
            }
        }
        const uint64_t any = __ballot(sp);
        if (lane == 0) sh.flag[wave] = any != 0;
    }
    __syncthreads();
    if (!vec || (sh.flag[0] | sh.flag[1] | sh.flag[2] | sh.flag[3])) {   // block-uniform
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const uint32_t x = tile_dword<DT>(rowp, false, nvalid, q);
            if constexpr (DT == SS_BF16) {
                const uint32_t lo = local_of(q, 0) < nvalid ? ord16_canon(x) : 0u;
                const uint32_t hi = local_of(q, 1) < nvalid ? ord16_canon(x >> 16) : 0u;
                kk[q] = lo | (hi << 16);
            } else {
                kk[q] = local_of(q, 0) < nvalid ? ord32(canon(bitsf(x))) : 0u;
            }
        }
    }
    // screening key of element (q, h) shifted down by `sh` bits
    auto skey_shr = [&](int q, int h, int s) -> uint32_t {
        if constexpr (DT == SS_BF16) return h ? kk[q] >> (16 + s) : (kk[q] & 0xFFFFu) >> s;
        else return kk[q] >> (16 + s);
    };
    const int nzero = BN - nvalid;   // slots with no element: key 0, in bucket 0 while the prefix is 0

    // ---- fast screen: the same 6 + 10-bit radix select over the tile's
    // chunk maxima (one value per 16-byte chunk, an eighth (bf16) or a
    // quarter (fp32) of the elements) gives T0, the 16-bit screening key of
    // the 128th largest chunk maximum.  Those 128 maxima are distinct
    // elements, so the 128th best element's screening key is >= T0; only the
    // chunks whose maximum reaches T0 can hold elements that high, and their
    // elements >= T0 (usually a little over 128) go to the bitonic finish at
    // once.  Ties at 16-bit precision (more than 256 such elements), more
    // such chunks than the copy area holds, and tiles with fewer than 128
    // chunks take the element screen below. ----
    if (rx_fast_screen<DT>(P, row, tile, kk, sh, nvalid)) return;
    __syncthreads();   // the shared area is reused

    // ---- screen: the 6 most significant bits.  Every thread counts its own
    // elements in its own LDS column (no two threads touch one word, and a
    // wave's columns lie on distinct banks), then a reduction tree sums the
    // columns. ----
#pragma unroll
    for (int b = 0; b < RX_NB1; ++b) sh.col[b][tid] = 0u;
#pragma unroll
    for (int i = tid; i < RX_NB2; i += S1_THREADS) sh.hist[i] = 0u;
    // a wave's LDS operations run in issue order: its column is clear before
    // its increments land
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int h = 0; h < HALVES; ++h)
            __hip_atomic_fetch_add(&sh.col[skey_shr(q, h, 10)][tid], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __syncthreads();
    {
        // thread t sums bucket t / 4 over the columns 64 (t % 4) .. +63,
        // starting at a rotating offset so that a wave's reads spread over the banks
        const int b = tid >> 2, part = tid & 3;
        const uint4* src = (const uint4*)&sh.col[b][part * 64];
        uint32_t s = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint4 v = src[(i + b) & 15];
            s += v.x + v.y + v.z + v.w;
        }
        s += xor_lane<1>(s);
        s += xor_lane<2>(s);
        if (part == 0) sh.h1[b] = s;
    }
    __syncthreads();
    if (wave == 0) {
        // bucket counts from the top: lane l holds bucket 63 - l
        int c = (int)sh.h1[RX_NB1 - 1 - lane];
        if (lane == RX_NB1 - 1) c -= nzero;
        const int incl = wave_incl_scan(c);
        const uint64_t reach = __ballot(incl >= KMAX);
        const int l = reach ? __builtin_ctzll(reach) : 0;   // uniform
        const int cl = __builtin_amdgcn_readlane(c, l);
        if (lane == 0) {
            sh.sel[0] = reach ? RX_NB1 - 1 - l : -1;
            sh.sel[1] = __builtin_amdgcn_readlane(incl, l) - cl;   // strictly above the bucket
            sh.sel[2] = cl;
        }
    }
    __syncthreads();
    uint32_t thr16;   // candidates: screening key >= thr16
    int d1 = sh.sel[0];
    if (d1 < 0) {
        thr16 = 1u;   // fewer than 128 elements: all of them
    } else if (sh.sel[1] + sh.sel[2] <= RX_CAP) {
        thr16 = max((uint32_t)d1 << 10, 1u);   // the screen alone leaves few enough
    } else {
        // ---- refinement: the next 10 bits of the elements in bucket d1,
        // counted in one shared histogram (the other lanes add to spare
        // entries of their own, so that they neither branch nor contend) ----
        const int need = KMAX - sh.sel[1];
        const uint32_t lo = (uint32_t)d1 << 10;
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int h = 0; h < HALVES; ++h) {
                const uint32_t dg = skey_shr(q, h, 0) - lo;   // the digit, if below RX_NB2
                if (__ballot(dg < (uint32_t)RX_NB2))
                    __hip_atomic_fetch_add(&sh.hist[dg < (uint32_t)RX_NB2 ? dg : (uint32_t)(RX_NB2 + lane)], 1u,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        __syncthreads();
        // thread t holds buckets 1023 - 4t .. 1020 - 4t; a block scan from the
        // top finds the bucket where the count reaches `need`
        const uint4 v = *(const uint4*)&sh.hist[RX_NB2 - 4 - 4 * tid];
        uint32_t c3 = v.w, c2 = v.z, c1 = v.y, c0 = v.x;
        if (tid == S1_THREADS - 1 && d1 == 0) c0 -= nzero;
        const int s = (int)(c0 + c1 + c2 + c3);
        const int wincl = wave_incl_scan(s);
        if (lane == WAVE - 1) sh.wsum[wave] = wincl;
        __syncthreads();
        int before = wincl - s;
#pragma unroll
        for (int w = 0; w < S1_WAVES; ++w) before += w < wave ? sh.wsum[w] : 0;
        const int cs[4] = {(int)c3, (int)c2, (int)c1, (int)c0};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (before < need && before + cs[j] >= need) {   // exactly one (thread, j)
                sh.sel[0] = RX_NB2 - 1 - 4 * tid - j;
                sh.sel[1] = before;
                sh.sel[2] = cs[j];
            }
            before += cs[j];
        }
        __syncthreads();
        thr16 = max(lo + (uint32_t)sh.sel[0], 1u);
    }

    // ---- candidates as exact keys (value, then lower id), compacted in LDS ----
    auto is_cand = [&](int q, int h) -> bool {
        if constexpr (DT == SS_BF16) return skey_shr(q, h, 0) >= thr16;
        else return kk[q] >= (thr16 << 16);
    };
    int wc = 0;   // this wave's candidates (uniform)
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int h = 0; h < HALVES; ++h) wc += __builtin_popcountll(__ballot(is_cand(q, h)));
    if (lane == 0) sh.wsum[wave] = wc;
    __syncthreads();
    int total = 0, pos = 0;
#pragma unroll
    for (int w = 0; w < S1_WAVES; ++w) {
        pos += w < wave ? sh.wsum[w] : 0;
        total += sh.wsum[w];
    }
    if (total > RX_CAP) {   // block-uniform: heavy ties at 16-bit precision
        __syncthreads();    // the shared area is reused
        radix_tie_fallback<DT>(P, row, tile, shu.tile);
        return;
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int h = 0; h < HALVES; ++h) {
            const bool c = is_cand(q, h);
            const uint64_t m = __ballot(c);
            if (m) {   // wave-uniform; every lane writes, the non-candidates to the spare entries
                const uint32_t loc = (uint32_t)local_of(q, h);
                const int slot = c ? pos + lane_prefix(m) : RX_CAP + lane;
                if constexpr (DT == SS_BF16)
                    sh.keys[slot] = (Key)((skey_shr(q, h, 0) << 16) | (0xFFFFu - loc));
                else
                    sh.keys[slot] = (Key)(((uint64_t)kk[q] << 32) | (uint64_t)(0xFFFFFFFFu - loc));
                pos += __builtin_popcountll(m);
            }
        }
    __syncthreads();
    if (wave == 0) {
        const WList<Key> best = wave_top128(sh.keys, total);
        const int64_t o = ((int64_t)row * P.Zv + tile) * KMAX + lane;
        ((Key*)P.scratch)[o] = best.lo;
        ((Key*)P.scratch)[o + WAVE] = best.hi;
    }
}

}  // namespace ssd
