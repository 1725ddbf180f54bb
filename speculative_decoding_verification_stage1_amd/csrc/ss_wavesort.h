// Sorted lists of 128 keys held by one wave (two per lane: rank `lane` in
// lo, rank `lane + 64` in hi, descending) and the bitonic networks that
// build and merge them with cross-lane exchanges instead of LDS round trips
// and workgroup barriers.  Keys are unsigned (uint32 or uint64); larger is
// better.
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

// Compare-exchange with lane ^ J in both halves; the lane keeps the larger
// key where *_max is set.
template <int J, typename K>
__device__ __forceinline__ void cas_step(WList<K>& c, bool lo_max, bool hi_max) {
    const K plo = xor_key<J>(c.lo), phi = xor_key<J>(c.hi);
    c.lo = lo_max ? kmax(c.lo, plo) : kmin(c.lo, plo);
    c.hi = hi_max ? kmax(c.hi, phi) : kmin(c.hi, phi);
}

// Half-cleaners j = J .. 1 on both halves (descending).
template <int J = 32, typename K>
__device__ __forceinline__ void wave_half_clean(WList<K>& c) {
    const bool lower = (lane_id() & J) == 0;
    cas_step<J>(c, lower, lower);
    if constexpr (J > 1) wave_half_clean<J / 2>(c);
}

// j = 64 step: rank lane against rank lane + 64, the larger to lo.
template <typename K>
__device__ __forceinline__ void cas_64(WList<K>& c) {
    const K t = kmax(c.lo, c.hi);
    c.hi = kmin(c.lo, c.hi);
    c.lo = t;
}

template <typename K>
__device__ __forceinline__ K reverse_lanes(K v) {
    const int r = (WAVE - 1 - lane_id()) * 4;
    if constexpr (sizeof(K) == 8) {
        const uint32_t x = (uint32_t)__builtin_amdgcn_ds_bpermute(r, (int)(uint32_t)v);
        const uint32_t y = (uint32_t)__builtin_amdgcn_ds_bpermute(r, (int)(uint32_t)((uint64_t)v >> 32));
        return (K)(((uint64_t)y << 32) | x);
    } else {
        return (K)(uint32_t)__builtin_amdgcn_ds_bpermute(r, (int)(uint32_t)v);
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

// Bitonic sort (descending) of 128 keys.  Stage k sorts blocks of k keys,
// descending where (index & k) == 0 and ascending otherwise.
template <int KS, int J, typename K>
__device__ __forceinline__ void sort_substeps(WList<K>& c) {
    const int lane = lane_id();
    const bool lower = (lane & J) == 0;
    const bool dlo = (lane & KS) == 0;
    const bool dhi = ((lane + 64) & KS) == 0;
    cas_step<J>(c, lower == dlo, lower == dhi);
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

}  // namespace ssd
