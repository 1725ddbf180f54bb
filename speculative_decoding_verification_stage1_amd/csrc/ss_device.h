// Device-side building blocks of libss: order keys, Philox4x32-10, the
// fixed exp/log used by the epilogue, and small wave/block helpers.
//
// Everything here is compiled with -ffp-contract=off; every fused
// multiply-add is an explicit __builtin_fmaf so the arithmetic is the same
// IEEE binary32 sequence on every run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ss.h"

namespace ssd {

constexpr int KMAX = SS_KMAX;
constexpr int WAVE = 64;

// ---------------------------------------------------------------------------
// bit views
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t fbits(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __uint_as_float(u); }

constexpr uint32_t F32_MAX_BITS = 0x7F7FFFFFu;
constexpr uint32_t F32_PINF_BITS = 0x7F800000u;
constexpr uint32_t F32_NINF_BITS = 0xFF800000u;

// Canonical value: NaN -> -inf, +inf -> FLT_MAX, -0 -> +0.
__device__ __forceinline__ float canon(float z) {
    if (z != z) return bitsf(F32_NINF_BITS);
    if (z == bitsf(F32_PINF_BITS)) return bitsf(F32_MAX_BITS);
    if (z == 0.0f) return 0.0f;
    return z;
}

// Order-preserving unsigned key of a (non-NaN) float: larger value <=> larger key.
__device__ __forceinline__ uint32_t ord32(float f) {
    uint32_t b = fbits(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float unord32(uint32_t k) {
    return bitsf((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// bf16 raw pattern -> 16-bit order key of its canonical value.  NaN maps to
// the key of -inf, -0 to the key of +0.  +inf keeps its own key (0xFF80),
// which ranks above every finite bf16 and is read back as FLT_MAX.
__device__ __forceinline__ uint32_t ord16_canon(uint32_t h) {
    h &= 0xFFFFu;
    if ((h & 0x7FFFu) > 0x7F80u) h = 0xFF80u;     // NaN -> -inf
    if (h == 0x8000u) h = 0u;                      // -0 -> +0
    return (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
}
constexpr uint32_t K16_NINF = 0x007Fu;   // ord16(-inf)
constexpr uint32_t K16_PINF = 0xFF80u;   // ord16(+inf)

// 16-bit key -> the 32-bit key of the canonical fp32 value.
__device__ __forceinline__ uint32_t k16_to_k32(uint32_t k16) {
    if (k16 == K16_PINF) return ord32(bitsf(F32_MAX_BITS));
    return (k16 & 0x8000u) ? (k16 << 16) : ((k16 << 16) | 0xFFFFu);
}

__device__ __forceinline__ float widen_bf16(uint32_t h) { return bitsf((h & 0xFFFFu) << 16); }

// Global-memory view of a pointer: loads through it are global_load (vector
// memory only) instead of flat loads, which also hold the LDS counter.
typedef uint32_t vu32x4 __attribute__((ext_vector_type(4)));   // 16-byte load unit
// Fourth word of a raw buffer resource on this chip family: 32-bit data
// format, no swizzle, no per-lane index.
constexpr int BUF_DWORD3 = 0x00020000;

// Cache policy for data read exactly once (the logits and grammar words):
// the nt bit, so that the stream is not kept in the caches in place of data
// that are read again (tile lists, request records).  Measured on a cold
// 128 MiB read in 64 KiB workgroups: 24.3 us with it, 26.9 us without.
constexpr int LD_STREAM = 2;

// A buffer view of `bytes` bytes at `base` (uniform).  Loads at offsets
// past the end return zero and touch no memory, so a fixed run of loads
// needs no branch around the ones that fall outside.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_view(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, BUF_DWORD3);
}
__device__ __forceinline__ uint32_t buf_u32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint64_t buf_u64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    return (uint64_t)v[0] | ((uint64_t)v[1] << 32);
}

// Data handed between workgroups of one launch.  Each XCD has its own L2,
// and a device-scope fence writes back or invalidates a whole L2 (µs each,
// serialised per XCD), so none is used: the producer writes with
// device-coherent stores (sc1: through to memory), waits until they have
// completed, then counts its arrival with a device-scope atomic (whose
// return value can carry the earlier producers' data as well); whoever sees
// the final count writes with device-coherent stores where earlier
// producers wrote, so that no cached copy is written back over its own.
template <typename T>
__device__ __forceinline__ void store_coherent(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's memory operations have completed (a compiler
// barrier as well).
__device__ __forceinline__ void wait_memory() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* gmem(const T* p) {
    return (const __attribute__((address_space(1))) T*)p;
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11): per round, words 0 and 2 are
// multiplied by the round constants, the high halves are mixed with words 1
// and 3 and the key, and the key advances by the Weyl increments.
// ---------------------------------------------------------------------------
struct u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ u32x4 philox10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        // each 32 x 32 -> 64 product as one multiply-add (both halves)
        const uint64_t pa = (uint64_t)0xD2511F53u * c.x, pb = (uint64_t)0xCD9E8D57u * c.z;
        const uint32_t a = (uint32_t)pa, ah = (uint32_t)(pa >> 32);
        const uint32_t b = (uint32_t)pb, bh = (uint32_t)(pb >> 32);
        c = u32x4{bh ^ c.y ^ k0, b, ah ^ c.w ^ k1, a};
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

// First output word for counter {c0, c1, c2, offset_lo} under key
// {seed_lo, seed_hi ^ offset_hi}.
__device__ __forceinline__ uint32_t philox_w0(uint64_t seed, uint64_t offset, uint32_t c0,
                                              uint32_t c1, uint32_t c2) {
    u32x4 c{c0, c1, c2, (uint32_t)offset};
    return philox10(c, (uint32_t)seed, (uint32_t)(seed >> 32) ^ (uint32_t)(offset >> 32)).x;
}

// u in (0,1): top 23 bits of the word, centred in their cell.
__device__ __forceinline__ float unit_open(uint32_t w) {
    return ((float)(w >> 9) + 0.5f) * 0x1p-23f;
}

// ---------------------------------------------------------------------------
// Fixed exp / log.  exp: Cody-Waite reduction x = n ln2 + r with a two-part
// ln 2, degree-7 Taylor polynomial of e^r, scale by 2^n; arguments below -86
// give 0.  log: x = 2^e m, m in (sqrt(1/2), sqrt(2)], ln m = 2 atanh((m-1)/
// (m+1)) by its odd series to the 9th power.
// ---------------------------------------------------------------------------
// exp for x <= 0 or -inf (never NaN), the only arguments the epilogue has
// (x = v - max v); the cut below -86 is a select, not a branch.
__device__ __forceinline__ float exp_fixed_nonpos(float x) {
    const float xc = x < -86.0f ? -86.0f : x;
    const float n = __builtin_rintf(xc * 0x1.715476p+0f);
    float r = __builtin_fmaf(-n, 0x1.62e4p-1f, xc);
    r = __builtin_fmaf(-n, 0x1.7f7d1cp-20f, r);
    float p = __builtin_fmaf(0x1.a01a02p-13f, r, 0x1.6c16c2p-10f);
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return x < -86.0f ? 0.0f : __builtin_ldexpf(p, (int)n);
}

__device__ __forceinline__ float log_fixed(float x) {
    if (x != x || x < 0.0f) return bitsf(0x7FC00000u);
    if (x == 0.0f) return bitsf(F32_NINF_BITS);
    if (x == bitsf(F32_PINF_BITS)) return x;
    int e = -127;
    if (x < 0x1p-126f) {   // subnormal: scale into the normal range (exact)
        x *= 0x1p24f;
        e -= 24;
    }
    const uint32_t b = fbits(x);
    e += (int)(b >> 23);
    float m = bitsf((b & 0x007FFFFFu) | 0x3F800000u);
    if (m > 0x1.6a09e6p+0f) {
        m *= 0.5f;
        e += 1;
    }
    const float s = (m - 1.0f) / (m + 1.0f);
    const float s2 = s * s;
    float q = __builtin_fmaf(0x1.c71c72p-4f, s2, 0x1.24924ap-3f);
    q = __builtin_fmaf(q, s2, 0x1.99999ap-3f);
    q = __builtin_fmaf(q, s2, 0x1.555556p-2f);
    const float h = __builtin_fmaf(s * s2, q, s);
    const float ef = (float)e;
    return __builtin_fmaf(ef, 0x1.62e4p-1f, __builtin_fmaf(ef, 0x1.7f7d1cp-20f, h + h));
}

// log_fixed for a positive, normal, finite x (its special cases and the
// subnormal scaling never apply): the same operations, with no branch.
__device__ __forceinline__ float log_fixed_normal(float x) {
    const uint32_t b = fbits(x);
    int e = (int)(b >> 23) - 127;
    float m = bitsf((b & 0x007FFFFFu) | 0x3F800000u);
    const bool big = m > 0x1.6a09e6p+0f;
    m = big ? m * 0.5f : m;
    e += big ? 1 : 0;
    const float s = (m - 1.0f) / (m + 1.0f);
    const float s2 = s * s;
    float q = __builtin_fmaf(0x1.c71c72p-4f, s2, 0x1.24924ap-3f);
    q = __builtin_fmaf(q, s2, 0x1.99999ap-3f);
    q = __builtin_fmaf(q, s2, 0x1.555556p-2f);
    const float h = __builtin_fmaf(s * s2, q, s);
    const float ef = (float)e;
    return __builtin_fmaf(ef, 0x1.62e4p-1f, __builtin_fmaf(ef, 0x1.7f7d1cp-20f, h + h));
}

// u lies in [2^-24, 1 - 2^-24], so -ln u is positive and normal: both
// logarithms take the branch-free form.
__device__ __forceinline__ float gumbel_noise(uint64_t seed, uint64_t offset, uint32_t c0,
                                              uint32_t c1, uint32_t c2) {
    const float u = unit_open(philox_w0(seed, offset, c0, c1, c2));
    return -log_fixed_normal(-log_fixed_normal(u));
}

// n / d for uniform d > 0: d = 1 and powers of two (the usual tile counts and
// rows per request) skip the integer division sequence.
__device__ __forceinline__ int div_uniform(int n, int d) {
    if (d == 1) return n;
    if ((d & (d - 1)) == 0) return n >> __builtin_ctz((unsigned)d);
    return n / d;
}

// ---------------------------------------------------------------------------
// wave helpers (wave64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

// Number of lanes below this one whose bit is set in `bal`.
__device__ __forceinline__ int lane_prefix(uint64_t bal) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
}

// inclusive prefix sum over the wave
__device__ __forceinline__ int wave_incl_scan(int v) {
    const int l = lane_id();
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const int t = __shfl_up(v, o, WAVE);
        if (l >= o) v += t;
    }
    return v;
}

// ---------------------------------------------------------------------------
// lane exchange v(lane ^ J) with no LDS traffic (every DPP pattern here is a
// full permutation, so bound_ctrl, which lets the compiler fold the move
// into the instruction that uses it, changes no value): DPP quad permutes for J =
// 1, 2; two DPP mirrors for J = 4 (quad reversal, then the 8-lane mirror:
// l ^ 3 ^ 7 = l ^ 4) and J = 8 (8-lane mirror, then the 16-lane mirror:
// l ^ 7 ^ 15 = l ^ 8); the gfx950 row-swap permutes for J = 16, 32.
// ---------------------------------------------------------------------------
constexpr int DPP_QUAD_REV = 0x1B;      // quad_perm [3,2,1,0]
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;

template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
    if constexpr (J == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
    } else if constexpr (J == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);
    } else if constexpr (J == 4) {
        const int a = __builtin_amdgcn_mov_dpp((int)v, DPP_QUAD_REV, 0xF, 0xF, true);
        return (uint32_t)__builtin_amdgcn_mov_dpp(a, DPP_ROW_HALF_MIRROR, 0xF, 0xF, true);
    } else if constexpr (J == 8) {
        const int a = __builtin_amdgcn_mov_dpp((int)v, DPP_ROW_HALF_MIRROR, 0xF, 0xF, true);
        return (uint32_t)__builtin_amdgcn_mov_dpp(a, DPP_ROW_MIRROR, 0xF, 0xF, true);
    } else if constexpr (J == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane_id() & 16) ? r[0] : r[1];
    } else {
        static_assert(J == 32, "xor distance");
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane_id() & 32) ? r[0] : r[1];
    }
}

template <int J>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v) {
    return ((uint64_t)xor_lane<J>((uint32_t)(v >> 32)) << 32) | xor_lane<J>((uint32_t)v);
}

}  // namespace ssd
