// Single-program-per-row top-k by MSB-to-LSB radix select: the design the
// two-stage method replaces (SonicSampler section 3.1, "Top-k selection
// primitives": radix select walks the key's digits from the most
// significant down, narrowing to the bucket that holds the k-th key;
// section 3.2: one program per row caps the parallelism at B programs).
//
// One workgroup streams its whole row once per pass.  Pass p histograms
// digit p (8 bits) of the order key of every element whose higher digits
// equal those of the k-th key found so far, and the bucket holding the k-th
// key extends that prefix.  As soon as the elements at or above the current
// prefix number at most RR_CAP, one more pass gathers them as exact 64-bit
// keys (order key, then lower id first) and a sort finishes the row.  When
// every digit is resolved and more elements than that still tie at the
// k-th value, a second radix select over the token index picks the lowest
// ids among the ties.
#pragma once

#include "ss_stage1.h"

namespace ssd {

constexpr int RR_THREADS = 256;
constexpr int RR_WAVES = RR_THREADS / WAVE;
constexpr int RR_CAP = 1024;   // candidates gathered for the final sort

struct RowRadixShared {
    uint32_t hist[RR_WAVES][256];   // per-wave digit counts
    uint32_t tot[256];              // their sum
    uint64_t cand[RR_CAP];          // candidate keys
    int ctr;
    int sel[2];                     // chosen bucket, elements above it
};

// Order key of element i of the row: uint32 ord32 of the canonical value
// (fp32), uint16 ord16 of the canonical bf16 value (NaN as -inf, -0 as +0).
template <int DT>
__device__ __forceinline__ uint32_t rr_key(uint32_t raw) {
    if constexpr (DT == SS_BF16) return ord16_canon(raw);
    else return ord32(canon(bitsf(raw)));
}
// Exact 64-bit key: the 32-bit order key of the canonical fp32 value, then
// the lower id first.
template <int DT>
__device__ __forceinline__ uint64_t rr_key64(uint32_t u, int id) {
    const uint32_t k32 = DT == SS_BF16 ? k16_to_k32(u) : u;
    return ((uint64_t)k32 << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}

// Calls f(id, raw) for every element of the row, the workgroup streaming
// it with 16-byte loads in row order (element by element for rows that do
// not start on a 16-byte boundary).
template <int DT, typename F>
__device__ __forceinline__ void rr_stream(const char* rowp, int V, bool aligned, F&& f) {
    constexpr int EPL = DT == SS_BF16 ? 8 : 4;   // elements per 16 bytes
    const int tid = threadIdx.x;
    if (aligned) {
        const int nvec = V / EPL;
        const __amdgpu_buffer_rsrc_t rs = buf_view(rowp, (uint32_t)nvec * 16u);
        constexpr int U = 16;   // loads in flight per thread: one workgroup per row must hide the latency alone
        for (int c0 = 0; c0 < nvec; c0 += U * RR_THREADS) {
            vu32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (c0 + u * RR_THREADS + tid) * 16, 0, LD_STREAM);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * RR_THREADS + tid;
                if (c < nvec) {
                    const uint32_t d[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                    for (int e = 0; e < EPL; ++e)
                        f(c * EPL + e, DT == SS_BF16 ? (d[e >> 1] >> (16 * (e & 1))) & 0xFFFFu : d[e]);
                }
            }
        }
        for (int i = nvec * EPL + tid; i < V; i += RR_THREADS)   // the ragged tail
            f(i, DT == SS_BF16 ? (uint32_t)gmem((const uint16_t*)rowp)[i] : gmem((const uint32_t*)rowp)[i]);
    } else {
        for (int i = tid; i < V; i += RR_THREADS)
            f(i, DT == SS_BF16 ? (uint32_t)gmem((const uint16_t*)rowp)[i] : gmem((const uint32_t*)rowp)[i]);
    }
}

// hist[wave][bin] += 1 for this lane's bin (valid lanes only).  Plain LDS
// adds: the LDS resolves lanes adding to one address far faster than a
// per-bin ballot loop (measured 4.6x on the 512 x 2^18 fp32 workload).
__device__ __forceinline__ void rr_count(uint32_t* h, uint32_t bin, bool valid) {
    if (valid) atomicAdd(&h[bin], 1u);
}

// Bucket of the kneed-th largest counted element from sh.tot (bins high to
// low): sel[0] = the bucket, sel[1] = elements in buckets above it.  Wave 0
// only; the caller synchronises.
__device__ __forceinline__ void rr_pick(RowRadixShared& sh, int kneed, bool from_top) {
    const int lane = lane_id();
    // lane l: bins 4l..4l+3 (from the top: bins 255-4l .. 252-4l)
    int s4[4], s = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int bin = from_top ? 255 - (4 * lane + k) : 4 * lane + k;
        s4[k] = (int)sh.tot[bin];
        s += s4[k];
    }
    const int pre = wave_incl_scan(s);                // bins ranked before and with this lane's
    const uint64_t ok = __ballot(pre >= kneed);
    const int L = __builtin_ctzll(ok);                // first lane reaching kneed
    int acc = __shfl(pre - s, L, WAVE);
    const int t0 = __shfl(s4[0], L, WAVE), t1 = __shfl(s4[1], L, WAVE), t2 = __shfl(s4[2], L, WAVE);
    int k;
    if (acc + t0 >= kneed) k = 0;
    else if (acc + t0 + t1 >= kneed) { k = 1; acc += t0; }
    else if (acc + t0 + t1 + t2 >= kneed) { k = 2; acc += t0 + t1; }
    else { k = 3; acc += t0 + t1 + t2; }
    if (lane == 0) {
        const int r = 4 * L + k;
        sh.sel[0] = from_top ? 255 - r : r;
        sh.sel[1] = acc;
    }
}

// The k best elements of one row (k <= 128) into wave 0's registers, sorted (key: 32-bit order key of the canonical fp32 value,
// then the lower id; 0 past the row's length).  `stream(f)` must call
// f(i, raw) once for every element i in [0, V) of the row (raw: the bf16
// pattern or the fp32 bits), across the workgroup, the same values on every
// call; it is called once per pass.  The whole workgroup calls this.
template <int DT, typename Stream>
__device__ __forceinline__ WList<uint64_t> radix_row_select(Stream&& stream, int V, int k, RowRadixShared& sh) {
    const int tid = threadIdx.x;
    const int wave = tid / WAVE;
    const int lane = lane_id();
    constexpr int KB = DT == SS_BF16 ? 16 : 32;
    const int K = min(k, V);

    auto clear_hist = [&] {
#pragma unroll
        for (int w = 0; w < RR_WAVES; ++w) sh.hist[w][tid] = 0u;
    };
    auto sum_hist = [&] {   // after a barrier; ends with one
        uint32_t t = 0;
#pragma unroll
        for (int w = 0; w < RR_WAVES; ++w) t += sh.hist[w][tid];
        sh.tot[tid] = t;
        __syncthreads();
    };

    // ---- value digits, most significant first ----
    uint32_t prefix = 0;   // the digits of the K-th key found so far
    int shift = KB;        // bits below the prefix
    int kneed = K;         // elements still wanted among those with this prefix
    int above = 0;         // elements above the prefix, all taken
    bool gathered = false;
    while (shift > 0) {    // block-uniform
        const int sft = shift - 8;
        clear_hist();
        __syncthreads();
        stream([&](int i, uint32_t raw) {
            const uint32_t u = rr_key<DT>(raw);
            const bool in = shift >= KB || (u >> shift) == prefix;
            rr_count(sh.hist[wave], (u >> sft) & 255u, in);
        });
        __syncthreads();
        sum_hist();
        if (wave == 0) rr_pick(sh, kneed, true);
        __syncthreads();
        const int b = sh.sel[0], ab = sh.sel[1];
        const int cnt_b = (int)sh.tot[b];
        prefix = (prefix << 8) | (uint32_t)b;
        shift = sft;
        above += ab;
        kneed -= ab;
        __syncthreads();   // sel and tot read before they change
        if (above + cnt_b <= RR_CAP) {   // gather every element at or above the prefix
            if (tid == 0) sh.ctr = 0;
            __syncthreads();
            stream([&](int i, uint32_t raw) {
                const uint32_t u = rr_key<DT>(raw);
                if ((u >> shift) >= prefix) sh.cand[atomicAdd(&sh.ctr, 1)] = rr_key64<DT>(u, i);
            });
            gathered = true;
            break;
        }
    }
    if (!gathered) {
        // every digit resolved: the K-th value's key is `prefix`; the
        // elements above it (fewer than K) and the kneed lowest ids among
        // those equal to it.  Radix select over the token index, low ids
        // first (24 bits cover any row).
        if (tid == 0) sh.ctr = 0;
        uint32_t ipre = 0;
        int ish = 24;
        int ineed = kneed;
        while (ish > 0) {
            const int sft = ish - 8;
            clear_hist();
            __syncthreads();
            stream([&](int i, uint32_t raw) {
                const bool in = rr_key<DT>(raw) == prefix && (ish >= 24 || ((uint32_t)i >> ish) == ipre);
                rr_count(sh.hist[wave], ((uint32_t)i >> sft) & 255u, in);
            });
            __syncthreads();
            sum_hist();
            if (wave == 0) rr_pick(sh, ineed, false);
            __syncthreads();
            ipre = (ipre << 8) | (uint32_t)sh.sel[0];
            ineed -= sh.sel[1];
            ish = sft;
            __syncthreads();
        }
        // ipre: the kneed-th lowest id among the ties
        stream([&](int i, uint32_t raw) {
            const uint32_t u = rr_key<DT>(raw);
            if (u > prefix || (u == prefix && (uint32_t)i <= ipre)) sh.cand[atomicAdd(&sh.ctr, 1)] = rr_key64<DT>(u, i);
        });
    }
    __syncthreads();
    // ---- sort the candidates: each wave folds its share of 128-key blocks,
    // then a merge tree over the waves ----
    const int n = min(sh.ctr, RR_CAP);
    WList<uint64_t> mine{0ull, 0ull};
    for (int c0 = wave * KMAX; c0 < n; c0 += RR_WAVES * KMAX) {
        const int i0 = c0 + lane, i1 = i0 + WAVE;
        WList<uint64_t> l{i0 < n ? sh.cand[i0] : 0ull, i1 < n ? sh.cand[i1] : 0ull};
        l = wave_sort128(l);
        mine = c0 == wave * KMAX ? l : wave_merge(mine, l);
    }
    __syncthreads();   // every wave has read its candidates
    sh.cand[wave * KMAX + lane] = mine.lo;
    sh.cand[wave * KMAX + lane + WAVE] = mine.hi;
    __syncthreads();
    if (wave < 2) {
        const WList<uint64_t> o{sh.cand[(wave + 2) * KMAX + lane], sh.cand[(wave + 2) * KMAX + lane + WAVE]};
        mine = wave_merge(mine, o);
        if (wave == 1) {
            sh.cand[KMAX * 1 + lane] = mine.lo;
            sh.cand[KMAX * 1 + lane + WAVE] = mine.hi;
        }
    }
    __syncthreads();
    if (wave == 0) {
        const WList<uint64_t> o{sh.cand[KMAX + lane], sh.cand[KMAX + lane + WAVE]};
        mine = wave_merge(mine, o);
        // ranks past K hold no element
        if (lane >= K) mine.lo = 0ull;
        if (lane + WAVE >= K) mine.hi = 0ull;
    }
    __syncthreads();   // the candidate area may be reused
    return mine;
}

template <int DT>
__global__ __launch_bounds__(RR_THREADS) void topk_radix_row_kernel(const void* logits, int V, int64_t ld,
                                                                    int aligned, int k, int32_t* out_ids,
                                                                    float* out_vals) {
    __shared__ RowRadixShared sh;
    const int row = blockIdx.x;
    const char* rowp = (const char*)logits + (int64_t)row * ld * (DT == SS_BF16 ? 2 : 4);
    const WList<uint64_t> best = radix_row_select<DT>(
        [&](auto&& f) { rr_stream<DT>(rowp, V, aligned != 0, f); }, V, k, sh);
    if (threadIdx.x < WAVE) {
        const int lane = lane_id();
        for (int h = 0; h < 2; ++h) {
            const int r = lane + WAVE * h;
            const uint64_t key = h ? best.hi : best.lo;
            if (r < k) {
                const bool have = key != 0ull;
                out_ids[(int64_t)row * k + r] = have ? (int)(0xFFFFFFFFu - (uint32_t)key) : -1;
                if (out_vals)
                    out_vals[(int64_t)row * k + r] = have ? unord32((uint32_t)(key >> 32)) : bitsf(F32_NINF_BITS);
            }
        }
    }
}

}  // namespace ssd
