// Sorted lists of 128 keys held by one wave (two per lane: rank `lane` in
// lo, rank `lane + 64` in hi, descending) and the bitonic networks that
// build and merge them with cross-lane exchanges instead of LDS round trips
// and workgroup barriers.  Keys are unsigned (uint32 or uint64); larger is
// better.
//
// A compare-exchange with lane ^ J keeps the larger key in some lanes and
// the smaller in the others; which lanes do depends only on J and the stage,
// so it is a compile-time 64-bit lane mask, turned into a per-lane flag with
// no vector instruction (inverse ballot).  For 32-bit keys within a row of
// 16 lanes a step is a max and a min that read the exchanged value through
// DPP, and one select; otherwise one exchange, one compare and one select.
#pragma once

#include "ss_device.h"

namespace ssd {

template <typename K>
struct WList {
    K lo, hi;
};

template <int J, typename K>
__device__ __forceinline__ K xor_key(K v) {
    if constexpr (sizeof(K) == 8) return (K)xor_lane64<J>((uint64_t)v);
    else return (K)xor_lane<J>((uint32_t)v);
}

template <typename K>
__device__ __forceinline__ K kmax(K a, K b) { return a > b ? a : b; }
template <typename K>
__device__ __forceinline__ K kmin(K a, K b) { return a < b ? a : b; }

// Lanes l (0..63) of a 64-key block at index offset `off` that keep the
// larger key at exchange distance J in a stage sorting blocks of KS keys,
// descending where (index & KS) == 0.
constexpr uint64_t keep_max_mask(int J, int KS, int off) {
    uint64_t m = 0;
    for (int l = 0; l < 64; ++l)
        if (((l & J) == 0) == (((l + off) & KS) == 0)) m |= 1ull << l;
    return m;
}

template <int J, uint64_t KEEP, typename K>
__device__ __forceinline__ K cas_lane(K a) {
    const K p = xor_key<J>(a);
    const bool keep_max = __builtin_amdgcn_inverse_ballot_w64(KEEP);
    if constexpr (sizeof(K) == 4 && J <= 8) {
        // 32-bit keys within a row of 16 lanes: max and min take the lane
        // exchange as an operand, and the lane mask picks one (no compare)
        return keep_max ? kmax(a, p) : kmin(a, p);
    } else {
        return ((p > a) == keep_max) ? p : a;
    }
}

// Half-cleaners j = J .. 1 on both halves (descending).
template <int J = 32, typename K>
__device__ __forceinline__ void wave_half_clean(WList<K>& c) {
    constexpr uint64_t M = keep_max_mask(J, 128, 0);   // lower lane of each pair keeps the max
    c.lo = cas_lane<J, M>(c.lo);
    c.hi = cas_lane<J, M>(c.hi);
    if constexpr (J > 1) wave_half_clean<J / 2>(c);
}

// j = 64 step: rank lane against rank lane + 64, the larger to lo.
template <typename K>
__device__ __forceinline__ void cas_64(WList<K>& c) {
    const K t = kmax(c.lo, c.hi);
    c.hi = kmin(c.lo, c.hi);
    c.lo = t;
}

// v(63 - lane): the 16-lane mirror (l ^ 15), then rows swapped by the
// row-swap permutes (l ^ 48).
__device__ __forceinline__ uint32_t reverse_lanes32(uint32_t v) {
    const uint32_t m = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, DPP_ROW_MIRROR, 0xF, 0xF, true);
    return xor_lane<16>(xor_lane<32>(m));
}
template <typename K>
__device__ __forceinline__ K reverse_lanes(K v) {
    if constexpr (sizeof(K) == 8) {
        const uint32_t x = reverse_lanes32((uint32_t)v);
        const uint32_t y = reverse_lanes32((uint32_t)((uint64_t)v >> 32));
        return (K)(((uint64_t)y << 32) | x);
    } else {
        return (K)reverse_lanes32((uint32_t)v);
    }
}

// The 128 best of two sorted lists, sorted: max(A[i], B[127-i]) is bitonic
// and holds them; the half-cleaners j = 64 .. 1 sort it.
template <typename K>
__device__ __forceinline__ WList<K> wave_merge(const WList<K>& a, const WList<K>& b) {
    WList<K> c;
    c.lo = kmax(a.lo, reverse_lanes(b.hi));
    c.hi = kmax(a.hi, reverse_lanes(b.lo));
    cas_64(c);
    wave_half_clean(c);
    return c;
}

// Bitonic sort (descending) of 128 keys.  Stage KS sorts blocks of KS keys,
// descending where (index & KS) == 0 and ascending otherwise.
template <int KS, int J, typename K>
__device__ __forceinline__ void sort_substeps(WList<K>& c) {
    c.lo = cas_lane<J, keep_max_mask(J, KS, 0)>(c.lo);
    c.hi = cas_lane<J, keep_max_mask(J, KS, 64)>(c.hi);
    if constexpr (J > 1) sort_substeps<KS, J / 2>(c);
}
template <int KS = 2, typename K>
__device__ __forceinline__ void sort_stages(WList<K>& c) {
    sort_substeps<KS, KS / 2>(c);
    if constexpr (KS < 64) sort_stages<KS * 2>(c);
}
template <typename K>
__device__ __forceinline__ WList<K> wave_sort128(WList<K> c) {
    sort_stages(c);   // lo descending, hi ascending: one bitonic sequence
    cas_64(c);
    wave_half_clean(c);
    return c;
}

// Bitonic sort (descending) of 64 keys, one per lane.
template <int KS, int J, typename K>
__device__ __forceinline__ void sort64_substeps(K& v) {
    v = cas_lane<J, keep_max_mask(J, KS, 0)>(v);
    if constexpr (J > 1) sort64_substeps<KS, J / 2>(v);
}
template <int KS = 2, typename K>
__device__ __forceinline__ void wave_sort64(K& v) {
    sort64_substeps<KS, KS / 2>(v);
    if constexpr (KS < 64) wave_sort64<KS * 2>(v);
}

}  // namespace ssd
