// LM head fused with the sampler's first stage (the fused sampling kernels
// the SonicSampler paper's related work names: the vocabulary projection
// and sampling in one pass, so that the logits never reach memory).
//
// logits[b, v] = sum_d H[b, d] * W[v, d]: H [B, D] and W [V, D] bf16, both
// K-contiguous; fp32 accumulation on the matrix cores
// (v_mfma_f32_32x32x16_bf16, k ascending in steps of 16; lane l of an
// operand holds row or column l % 32 and the 8 consecutive k at 8 * (l /
// 32) of the step).  Every launch shape below issues that same sequence for
// every output, so a logit has the same fp32 value whichever launch
// computes it.
//
// GEMM: a workgroup of 4 waves owns MT = 64 * WM rows and NT = (4 / WM) *
// 32 * WN vocabulary columns; a wave owns 64 rows x 32 * WN columns as
// 2 x WN blocks of 32 x 32.  The k loop runs in stages of KB (64 or 128):
// the stage's H and W rows go straight from global memory to one of two or
// three LDS stage buffers (16-byte direct loads, two stages ahead where
// three buffers fit), whose 16-byte slots are XOR-swizzled by row, so the
// fragment reads (32 rows at one k offset) meet no bank conflicts.  When
// several row blocks share
// a column tile, the blocks of one tile are given ids 8 apart, which the
// dispatcher places on the same XCD: the second read of a W tile then
// comes from that XCD's L2.
//
// The sampled result must be the bounded sampler applied to these logits,
// so the epilogue keeps every token that can be among a row's 128 best:
//  1. a probe launch computes the first P columns (whole fp32 tiles of
//     16384, at least one and V / 16) into the workspace, and the fp32 tile stage gives each row the exact
//     128 best of each probe tile; the largest of the tiles' 128th values
//     is a lower bound theta on the row's 128th best over the whole
//     vocabulary (any subset's k-th largest is at most the whole set's);
//  2. the main launch computes the other columns, and its epilogue appends
//     every token whose value exceeds theta (a tie with theta ranks below it:
//     higher id) to the row's candidate list - about (V/P - 1) * 128 tokens
//     per row - with its exact merge key;
//  3. the fused Stage 2 merges the probe lists with the sorted candidates
//     and runs the sampling epilogue.
// A row with more candidates than the list holds (inputs tied or peaked far
// from the probe columns) is handled by a third launch of the GEMM between
// 2 and 3: its workgroups return at once unless one of their rows
// overflowed, and otherwise store those columns' logits to the workspace,
// where Stage 2 radix-selects the row.
#pragma once

#include "ss_stage2.h"
#include "ss_radix_row.h"

namespace ssd {

constexpr int LM_CAP = 4096;     // candidates kept per row
#ifndef LM_S2_PF
#define LM_S2_PF 6
#endif
constexpr int LM_PROBE_MIN = 16384;

enum { LM_STORE = 0, LM_THRESH = 1, LM_REDO = 2 };

typedef __bf16 lm_bf16x8 __attribute__((ext_vector_type(8)));
typedef float lm_f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int lm_u32x4 __attribute__((ext_vector_type(4)));

struct LmParams {
    const uint16_t* H;
    int64_t ldh;
    const uint16_t* W;
    int64_t ldw;
    int B, D, V;
    int col_begin, col_end;        // columns this launch covers
    int ncol_tiles, nrow_tiles;    // tiles of this launch's shape
    float* out;                    // LM_STORE, LM_REDO: [B, ldo] logits of columns col_begin..
    int64_t ldo;
    const uint64_t* probe_keys;    // LM_THRESH: the probe tiles' sorted 128 per row ([B][Zp][128] fp32 tile keys)
    int Zp;
    uint64_t* cand;                // LM_THRESH: [B, LM_CAP] merge keys
    int32_t* cnt;                  // LM_THRESH, LM_REDO: [B] candidates appended (may exceed LM_CAP)
};

// workgroup id -> (column tile, row tile): the row tiles of one column tile
// get ids 8 apart (the same XCD under round-robin dispatch)
__device__ __forceinline__ bool lm_tile(const LmParams& p, int& ct, int& rt) {
    const int L = blockIdx.x;
    if (p.nrow_tiles == 1) {
        ct = L;
        rt = 0;
    } else {
        const int g = L / (8 * p.nrow_tiles), i = L % (8 * p.nrow_tiles);
        ct = g * 8 + (i & 7);
        rt = i >> 3;
    }
    return ct < p.ncol_tiles;
}

// Workgroup: WM x WNW = 4 waves multiply, each a tile of 64 rows by 32 WN
// columns; with SPLIT, four more waves only issue the global loads (so that
// a wave stalled on issuing a load never holds up the multiplies).  NTW:
// the weight rows are read with the nt policy (a launch with one row tile
// reads each weight once; the hidden rows, read by every workgroup, then
// stay in L2).
template <int MODE, int WM, int WNW, int WN, int KB, bool SPLIT, bool NTW>
__global__ __launch_bounds__((WM * WNW + (SPLIT ? 4 : 0)) * WAVE) void lmhead_gemm_kernel(LmParams p) {
    constexpr int NWC = WM * WNW;               // multiplying waves
    constexpr int NTC = NWC * WAVE;             // their threads
    constexpr int NTH = NTC + (SPLIT ? 4 * WAVE : 0);
    constexpr int NWL = SPLIT ? 4 : NWC;        // waves issuing the loads
    constexpr int MT = 64 * WM;                 // rows per workgroup
    constexpr int NT = WNW * 32 * WN;           // columns per workgroup
    constexpr int CPR = KB / 8;                 // 16-byte chunks per row and stage
    constexpr int SROW = KB * 2;                // LDS bytes per row and stage
    constexpr int AB = MT * SROW, WB = NT * SROW;
    static_assert(KB % 16 == 0 && NWC == 4, "tile shape");
    // LDS stages: NST buffers of (A tile | W tile), each row's 16-byte
    // chunks XOR-swizzled (slot below).  The global loads write LDS
    // directly (global_load_lds_dwordx4: each wave instruction fills 1 KiB,
    // lane L at byte 16 L of it, so lane L loads the chunk that the swizzle
    // puts there), NST - 1 stages ahead of the one being multiplied: no
    // registers stage the data and nothing waits for a load issued one
    // stage earlier.  The buffers are separate arrays, used in a fixed
    // rotation, so the compiler sees which one each LDS read touches and
    // does not wait for the loads in flight to the others.
    // Two stages when two workgroups' pairs fit in a CU's 160 KiB (the
    // 64-row tiles, whose registers also allow two workgroups per CU: one
    // workgroup's multiplies then cover the other's loads), else three when
    // they fit, else two.  Measured at B=64, D=4096, V=2^17: 203 us with
    // two stages and two workgroups per CU, 263 us with three stages and one.
    constexpr int LDS_CU = 160 * 1024;
    constexpr int NST = 4 * (AB + WB) <= LDS_CU ? 2 : (3 * (AB + WB) <= LDS_CU - 16 * 1024 ? 3 : 2);
    constexpr int RPI = 1024 / SROW;                      // rows one wave instruction fills
    constexpr int NINS = (MT + NT) / RPI;                 // instructions per stage
    constexpr int LPW = NINS / NWL;                       // per loading wave
    static_assert(1024 % SROW == 0 && MT % RPI == 0 && NT % RPI == 0 && NINS % NWL == 0, "direct loads");
    static_assert((NST - 2) * LPW <= 63 && LPW <= 63, "vmcnt range");
    static_assert((MT / RPI) % NWL == 0, "each loading wave's first instructions are the A rows");
    __shared__ __attribute__((aligned(16))) unsigned char lds0[AB + WB];
    __shared__ __attribute__((aligned(16))) unsigned char lds1[AB + WB];
    __shared__ __attribute__((aligned(16))) unsigned char lds2[NST > 2 ? AB + WB : 16];
    unsigned char* const bufs[3] = {lds0, lds1, lds2};
    int ct, rt;
    if (!lm_tile(p, ct, rt)) return;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int lane = lane_id();
    const bool loader = SPLIT && wave >= NWC;   // SPLIT: the last four waves issue the loads
    const int lwave = SPLIT ? (loader ? wave - NWC : 0) : wave;   // index among the loading waves
    const int row0 = rt * MT;
    const int col0 = p.col_begin + ct * NT;
    if (MODE == LM_REDO) {   // only blocks holding an overflowed row go on
        bool over = false;
        for (int i = tid; i < MT; i += NTH) {
            const int r = row0 + i;
            over |= r < p.B && p.cnt[r] > LM_CAP;
        }
        if (!__syncthreads_or(over)) return;
    }
    // slot of chunk c of row r: c ^ f(r), with f chosen so that the 16
    // rows one 16-lane phase of a fragment read touches (and the rows one
    // load instruction writes) land on distinct 16-byte bank groups of a
    // 256-byte window, and any 8 consecutive rows on distinct groups of a
    // 128-byte one
    auto swz = [](int r) {
        if constexpr (CPR >= 16) return r & 15;
        else if constexpr (CPR == 8) return (r & 7) ^ ((r >> 3) & 1);
        else return r & (CPR - 1);
    };
    auto slot = [&](int r, int c) { return r * SROW + 16 * (c ^ swz(r)); };
    // this lane's source for each of its wave's LPW instructions (rows past
    // the end read the last valid row; their results are dropped), and the
    // instruction's LDS offset in a stage buffer
    const uint16_t* src[LPW];
    int dst[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int ins = lwave + NWL * i;
        const bool is_a = ins < MT / RPI;
        const int rb = (is_a ? ins : ins - MT / RPI) * RPI;   // first row of the instruction's block
        const int r = rb + lane / CPR;
        const int c = (lane % CPR) ^ swz(r);                    // the chunk that lands at this lane's slot
        if (is_a) {
            const int g = row0 + r;
            src[i] = p.H + (int64_t)(g < p.B ? g : p.B - 1) * p.ldh + c * 8;
        } else {
            const int g = col0 + r;
            src[i] = p.W + (int64_t)(g < p.col_end ? g : p.col_end - 1) * p.ldw + c * 8;
        }
        dst[i] = (is_a ? 0 : AB) + rb * SROW;
    }
    auto issue = [&](int k0, unsigned char* buf) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const auto g = (const __attribute__((address_space(1))) void*)(src[i] + k0);
            const auto l = (__attribute__((address_space(3))) void*)(buf + dst[i]);
            if (NTW && i >= MT / RPI / NWL) __builtin_amdgcn_global_load_lds(g, l, 16, 0, LD_STREAM);
            else __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
        }
    };
    const int wr = (wave / WNW) * 64;            // this wave's rows and columns in the tile
    const int wc = (wave % WNW) * 32 * WN;
    lm_f32x16 acc[2][WN];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = lm_f32x16{};
    auto compute = [&](const unsigned char* buf) {
        const unsigned char* la = buf;
        const unsigned char* lw = buf + AB;
#pragma unroll
        for (int u = 0; u < KB / 16; ++u) {
            const int c = 2 * u + (lane >> 5);   // this lane's 16-byte chunk of the step
            lm_bf16x8 a[2], b[WN];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = __builtin_bit_cast(lm_bf16x8, *(const lm_u32x4*)(la + slot(wr + 32 * i + (lane & 31), c)));
#pragma unroll
            for (int j = 0; j < WN; ++j)
                b[j] = __builtin_bit_cast(lm_bf16x8, *(const lm_u32x4*)(lw + slot(wc + 32 * j + (lane & 31), c)));
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < WN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };
    // stage s: wait for this wave's loads of s (the loads of the stages
    // after it, at most NST - 2, may stay in flight), then a barrier - every
    // wave's part of s has landed and every wave is done with stage s - 1,
    // whose buffer the loads of s + NST - 1 then reuse.  The barrier is the
    // bare s_barrier: a workgroup fence would wait for every load in flight.
    auto barrier = [] {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    auto wait_stage = [&](bool last) {
        constexpr int VM = (NST - 2) * LPW;
        constexpr int ENC = (VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8);   // vmcnt(VM), others free
        if (last) __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0)
        else __builtin_amdgcn_s_waitcnt(ENC);
        barrier();
    };
    const int S = p.D / KB;
    // the loads of stage s + NST - 1 are issued unconditionally (past the
    // last stage they reload the last stage's data into a buffer no later
    // stage reads), so the loop body is straight-line code: a branch around
    // the loads would make the compiler wait for all of them before the
    // next LDS read.  The loop runs whole rotations of the buffers; the
    // last stages (fewer than NST, their loads issued already) follow it.
    if constexpr (!SPLIT) {
#pragma unroll
        for (int j = 0; j < NST - 1; ++j) issue((j < S ? j : S - 1) * KB, bufs[j]);
        int s0 = 0;
        for (; s0 + NST <= S; s0 += NST) {
#pragma unroll
            for (int j = 0; j < NST; ++j) {
                wait_stage(false);
                const int sn = s0 + j + NST - 1;
                issue((sn < S ? sn : S - 1) * KB, bufs[(j + NST - 1) % NST]);
                compute(bufs[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < NST - 1; ++j)
            if (s0 + j < S) {
                wait_stage(true);
                compute(bufs[j]);
            }
    } else if (loader) {
        // the same barriers as the multiplying waves, one per stage: wait
        // for this wave's loads of stage s, meet the others, then refill
        // the buffer of stage s - 1
#pragma unroll
        for (int j = 0; j < NST - 1; ++j) issue((j < S ? j : S - 1) * KB, bufs[j]);
        int s0 = 0;
        for (; s0 + NST <= S; s0 += NST) {
#pragma unroll
            for (int j = 0; j < NST; ++j) {
                wait_stage(false);
                const int sn = s0 + j + NST - 1;
                issue((sn < S ? sn : S - 1) * KB, bufs[(j + NST - 1) % NST]);
            }
        }
#pragma unroll
        for (int j = 0; j < NST - 1; ++j)
            if (s0 + j < S) wait_stage(true);
        __syncthreads();   // after its own loads have landed (the fence waits for them)
        return;            // a barrier waits only for the waves still running
    } else {
        int s0 = 0;
        for (; s0 + NST <= S; s0 += NST) {
#pragma unroll
            for (int j = 0; j < NST; ++j) {
                barrier();
                compute(bufs[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < NST - 1; ++j)
            if (s0 + j < S) {
                barrier();
                compute(bufs[j]);
            }
    }
    __syncthreads();   // every wave is done with the stage buffers, and every load has landed
    // THRESH: the rows' thresholds (the largest 128th key over the probe
    // tiles); then each wave appends the values above their row's
    // threshold to its own LDS list, slots given by a ballot prefix (no
    // atomic waits inside the compares: up to CAPW per wave, more go
    // straight to the row's global list); then the block counts its
    // candidates per row, one global atomic per row reserves the block's
    // share of the row's list, and the keys are written there.  (The stage
    // buffers are free after the k loop.)
    constexpr int NWAVES = NWC;
    constexpr int CAPW = 512;
    static_assert(NWAVES * CAPW * (8 + 2 + 2) + 3 * MT * 4 + 16 <= AB + WB, "candidate staging");
    static_assert(MT <= 65536, "row index in 16 bits");
    uint64_t* wkeys = (uint64_t*)&lds0[0];                    // [NWAVES][CAPW] keys
    uint16_t* wrow = (uint16_t*)(wkeys + NWAVES * CAPW);      // [NWAVES][CAPW] their rows in the tile
    uint16_t* wpos = wrow + NWAVES * CAPW;                    // [NWAVES][CAPW] their slots in the row's share
    uint32_t* theta = (uint32_t*)(wpos + NWAVES * CAPW);      // [MT]
    uint32_t* rcnt = theta + MT;                              // [MT]
    uint32_t* rbase = rcnt + MT;                              // [MT]
    uint32_t* wn = rbase + MT;                                // [NWAVES]
    if (MODE == LM_THRESH) {
        for (int i = tid; i < MT; i += NTC) {
            const int r = row0 + i;
            uint32_t t = 0xFFFFFFFFu;
            if (r < p.B) {
                t = 0u;
                for (int z = 0; z < p.Zp; ++z) {
                    const uint32_t k = (uint32_t)(p.probe_keys[((int64_t)r * p.Zp + z) * KMAX + (KMAX - 1)] >> 32);
                    t = k > t ? k : t;
                }
            }
            theta[i] = t;
            rcnt[i] = 0u;
        }
        __syncthreads();
    }
    // accumulator block (i, j), register q: row 32i + 8(q/4) + 4(l/32) + q%4,
    // column 32j + l%32 of this wave's.  THRESH: the thresholds of the
    // lane's 32 rows go to registers first, as floats: with t the key's
    // canonical value, ord32(canon(v)) > key holds exactly when v > t as
    // floats (NaN compares false and maps to -inf, -0 compares equal to +0
    // and maps to +0), except that +inf maps to FLT_MAX, so a threshold of
    // FLT_MAX becomes +inf; the key 0xFFFFFFFF of rows past B becomes a NaN
    // (no candidates).  Every probe tile is full, so its 128th key belongs
    // to a token and is at least the key of -inf.
    float thf[2][16];
    if (MODE == LM_THRESH) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const uint32_t t = theta[wr + 32 * i + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3)];
                const float f = unord32(t);
                thf[i][q] = f == bitsf(F32_MAX_BITS) ? bitsf(F32_PINF_BITS) : f;
            }
    }
    int nw = 0;   // THRESH: this wave's candidates so far (wave-uniform)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int rl = wr + 32 * i + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                const int r = row0 + rl;
                const int c = col0 + wc + 32 * j + (lane & 31);
                const bool in = r < p.B && c < p.col_end;
                const float v = acc[i][j][q];
                if (MODE != LM_THRESH) {
                    if (in) p.out[(int64_t)r * p.ldo + (c - p.col_begin)] = v;
                } else {
                    const bool cand = in && v > thf[i][q];
                    const uint64_t bal = __ballot(cand);
                    if (__builtin_expect(bal != 0ull, 0)) {   // wave-uniform; rare: kept out of line
                        if (cand) {
                            const uint32_t k32 = ord32(canon(v));
                            const uint64_t key = ((uint64_t)k32 << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)c);
                            const int pos = nw + lane_prefix(bal);
                            if (pos < CAPW) {
                                wkeys[wave * CAPW + pos] = key;
                                wrow[wave * CAPW + pos] = (uint16_t)rl;
                            } else {
                                const int at = atomicAdd(p.cnt + r, 1);
                                if (at < LM_CAP) p.cand[(int64_t)r * LM_CAP + at] = key;
                            }
                        }
                        nw += __popcll(bal);
                    }
                }
            }
    if (MODE == LM_THRESH) {
        if (lane == 0) wn[wave] = (uint32_t)(nw < CAPW ? nw : CAPW);
        __syncthreads();
        uint32_t nwv[NWAVES], tot = 0;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) {
            nwv[w] = wn[w];
            tot += nwv[w];
        }
        // entry e of the waves' lists, in wave order -> (wave, index)
        auto at_e = [&](uint32_t e) -> int {
            int w = 0;
#pragma unroll
            for (int u = 0; u < NWAVES - 1; ++u)
                if (w == u && e >= nwv[u]) {
                    e -= nwv[u];
                    w = u + 1;
                }
            return w * CAPW + (int)e;
        };
        for (uint32_t e = tid; e < tot; e += NTC) {
            const int x = at_e(e);
            wpos[x] = (uint16_t)atomicAdd(rcnt + wrow[x], 1u);
        }
        __syncthreads();
        for (int i = tid; i < MT; i += NTC)
            if (rcnt[i] > 0u) rbase[i] = (uint32_t)atomicAdd(p.cnt + row0 + i, (int)rcnt[i]);
        __syncthreads();
        for (uint32_t e = tid; e < tot; e += NTC) {
            const int x = at_e(e);
            const int i = wrow[x];
            const uint32_t at = rbase[i] + wpos[x];
            if (at < (uint32_t)LM_CAP) p.cand[(int64_t)(row0 + i) * LM_CAP + at] = wkeys[x];
        }
    }
}

// Fused Stage 2 for the LM head: one workgroup per row.
struct LmStage2Params {
    Stage2Params f;                // request records, outputs, generator copy (f.s1.V = the vocabulary)
    const uint64_t* probe_keys;    // [B][Zp][128] fp32 tile keys of columns 0 .. P-1
    int Zp;
    const uint64_t* cand;          // [B, LM_CAP]
    const int32_t* cnt;            // [B]
    const float* probe;            // [B, P] logits of columns 0 .. P-1
    const float* rest;             // [B, V - P] logits of columns P .. V-1 (overflowed rows only)
    int P;
};

union LmStage2Shared {
    S2Shared s2;
    RowRadixShared rr;
};

__global__ __launch_bounds__(S2_THREADS) void lmhead_stage2_kernel(LmStage2Params q) {
    __shared__ LmStage2Shared shu;
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const int wave = tid / WAVE;
    const int lane = lane_id();
    const Stage2Params& F = q.f;
    // the work items: the probe tiles' sorted lists, then the candidates in
    // chunks of 128, dealt to the waves in turn.  A wave's first LM_S2_PF
    // items are requested together with the count (their addresses stay
    // inside the row's probe keys and candidate area whatever the count;
    // entries past it are dropped once it is known), so that they cost one
    // round trip instead of one each (median of 15 launches, B=256, V=2^18:
    // 20.5 -> 19.1 us; B=64, V=2^17: 14.6 -> 14.0 us; the chunks' sorts and
    // merges are most of the rest)
    const uint64_t* c = q.cand + (int64_t)row * LM_CAP;
    const int n_raw = q.cnt[row];
    uint64_t pre[LM_S2_PF][2];
#pragma unroll
    for (int u = 0; u < LM_S2_PF; ++u) {
        const int it = wave + S2_WAVES * u;
        const bool isp = it < q.Zp;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int j = lane + WAVE * h;
            const int i = (it - q.Zp) * KMAX + j;
            const uint64_t* ptr = isp ? q.probe_keys + ((int64_t)row * q.Zp + it) * KMAX + j
                                      : c + (i < LM_CAP ? i : LM_CAP - 1);
            pre[u][h] = *ptr;
        }
    }
    const int n = __builtin_amdgcn_readfirstlane(n_raw);
    WL64 best{0ull, 0ull};
    if (n <= LM_CAP) {   // block-uniform
        const int items = q.Zp + (n + KMAX - 1) / KMAX;
        WL64 mine{0ull, 0ull};
        bool any = false;
        auto item = [&](int it, uint64_t k_lo, uint64_t k_hi) -> WL64 {
            if (it < q.Zp) return WL64{merge_key<SS_F32>(k_lo, it), merge_key<SS_F32>(k_hi, it)};
            const int i0 = (it - q.Zp) * KMAX + lane, i1 = i0 + WAVE;
            return wave_sort128(WL64{i0 < n ? k_lo : 0ull, i1 < n ? k_hi : 0ull});
        };
#pragma unroll
        for (int u = 0; u < LM_S2_PF; ++u) {
            const int it = wave + S2_WAVES * u;
            if (it < items) {
                const WL64 l = item(it, pre[u][0], pre[u][1]);
                mine = any ? wave_merge(mine, l) : l;
                any = true;
            }
        }
        for (int it = wave + S2_WAVES * LM_S2_PF; it < items; it += S2_WAVES) {
            const int i0 = (it - q.Zp) * KMAX + lane, i1 = i0 + WAVE;
            const WL64 l = item(it, it < q.Zp ? q.probe_keys[((int64_t)row * q.Zp + it) * KMAX + lane] : c[i0 < n ? i0 : 0],
                                it < q.Zp ? q.probe_keys[((int64_t)row * q.Zp + it) * KMAX + lane + WAVE] : c[i1 < n ? i1 : 0]);
            mine = any ? wave_merge(mine, l) : l;
            any = true;
        }
        S2Shared& sh = shu.s2;
        sh.wl[wave][0][lane] = mine.lo;
        sh.wl[wave][1][lane] = mine.hi;
        __syncthreads();
        auto wl = [&](int w) -> WL64 { return WL64{sh.wl[w][0][lane], sh.wl[w][1][lane]}; };
        if (wave == 1) {
            const WL64 z = wave_merge(wl(2), wl(3));
            sh.wl[2][0][lane] = z.lo;
            sh.wl[2][1][lane] = z.hi;
        }
        if (wave == 0) best = wave_merge(mine, wl(1));
        __syncthreads();
        if (wave == 0) best = wave_merge(best, wl(2));
    } else {
        // more candidates than the list holds: a radix select over the
        // row's stored logits
        const float* pr = q.probe + (int64_t)row * q.P;
        const float* rr = q.rest + (int64_t)row * (F.s1.V - q.P);
        best = radix_row_select<SS_F32>(
            [&](auto&& f) {
                for (int v = tid; v < q.P; v += S2_THREADS) f(v, fbits(pr[v]));
                for (int v = q.P + tid; v < F.s1.V; v += S2_THREADS) f(v, fbits(rr[v - q.P]));
            },
            F.s1.V, KMAX, shu.rr);
    }
    if (tid >= WAVE) return;
    const int b = row;
    ss_rng rg{0ull, 0ull};
    if (F.rng) rg = *F.rng;
    const RowParams rp = row_params(F.s1, b);
    VerifyPre vp{DraftCount{0, true}, -1};
    row_epilogue<SS_F32, MODE_SAMPLE>(F, rp, row, b, best, rg, shu.s2, vp);
}

}  // namespace ssd
