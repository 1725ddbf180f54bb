// libss: C ABI entry points (declared in include/ss.h).  Host code checks
// the arguments, carves the caller's workspace and queues fixed-grid
// kernels on the caller's stream; it never allocates or synchronises.
#include <mutex>

#include "ss_kernels.h"
#include "ss_dense.h"
#include "ss_radix.h"
#include "ss_radix_row.h"
#include "ss_lmhead.h"
#include "ss_listed_long.h"

using namespace ssd;

// The workspace of ss_sample_step_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: kernels receive the address that
// hipGetSymbolAddress returns for the current device (noalloc_scratch).
static __device__ __align__(256) unsigned char scratch[SS_NOALLOC_WS_BYTES];

namespace {

constexpr int KERNEL_ROWS_MAX = 1 << 24;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int tile_of(int dtype) { return dtype == SS_BF16 ? S1Traits<SS_BF16>::BN : S1Traits<SS_F32>::BN; }
size_t key_bytes(int dtype) { return dtype == SS_BF16 ? sizeof(uint32_t) : sizeof(uint64_t); }
int tiles_of(int V, int dtype) { return (V + tile_of(dtype) - 1) / tile_of(dtype); }

size_t scratch_bytes(int rows, int V, int dtype) {
    return align256((size_t)rows * (size_t)tiles_of(V, dtype) * KMAX * key_bytes(dtype));
}
size_t rec_bytes(int rows) { return align256((size_t)rows * sizeof(RowRec)); }
size_t listed_bytes(int rows) { return align256((size_t)rows * KMAX * sizeof(uint64_t)); }
constexpr size_t RNG_SNAP_BYTES = 256;
// Verification's per-request decision words (64 bits: arrivals and
// per-position bits), at the start of the workspace; each verification
// step zeroes its requests' words in its Stage-1 launch.
constexpr size_t ARRIVE_BYTES = 4096;
constexpr int ARRIVE_REQUESTS_MAX = (int)(ARRIVE_BYTES / sizeof(uint64_t));

// workspace: [arrival counters][tile keys][listed-token keys][row records
// or decisions][rng copy]
struct WsLayout {
    uint32_t* arrive;
    void* scratch;
    uint64_t* listed;
    RowRec* recs;
    ss_rng* rng_snap;
};
WsLayout ws_layout(void* ws, int rows, int V, int dtype) {
    WsLayout L;
    L.arrive = (uint32_t*)ws;
    L.scratch = (char*)ws + ARRIVE_BYTES;
    L.listed = (uint64_t*)((char*)L.scratch + scratch_bytes(rows, V, dtype));
    L.recs = (RowRec*)((char*)L.listed + listed_bytes(rows));
    L.rng_snap = (ss_rng*)((char*)L.recs + rec_bytes(rows));
    return L;
}

int check_logits(const void* logits, int dtype, int rows, int V, int64_t ld) {
    if (dtype != SS_F32 && dtype != SS_BF16) return SS_ERR_UNSUPPORTED;
    if (rows < 0 || V < 1 || ld < V) return SS_ERR_INVALID_ARG;
    if (V > SS_V_MAX || rows > KERNEL_ROWS_MAX) return SS_ERR_UNSUPPORTED;
    if (rows > 0 && !logits) return SS_ERR_INVALID_ARG;
    if ((int64_t)rows * tiles_of(V, dtype) > 0x7FFFFFFFLL) return SS_ERR_UNSUPPORTED;
    return SS_OK;
}

int check_aux(const ss_aux* aux, int V) {
    if (!aux) return SS_OK;
    if (aux->prior_stride < 0 || aux->bias_stride < 0 || aux->bitmask_stride < 0) return SS_ERR_INVALID_ARG;
    if (aux->bitmask && aux->bitmask_stride < ((int64_t)V + 31) / 32) return SS_ERR_INVALID_ARG;
    return SS_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return SS_OK;
    if (!ws || ws_bytes < need || ((uintptr_t)ws & 255u)) return SS_ERR_WORKSPACE;
    return SS_OK;
}

int aligned16(const void* logits, int dtype, int64_t ld) {
    const size_t es = dtype == SS_BF16 ? 2 : 4;
    return (((uintptr_t)logits & 15u) == 0) && (((size_t)ld * es) % 16 == 0);
}

ss_aux aux_or_empty(const ss_aux* aux) {
    ss_aux a{};
    if (aux) a = *aux;
    return a;
}

int launched() { return hipGetLastError() == hipSuccess ? SS_OK : SS_ERR_HIP; }

Stage1Params make_s1(const void* logits, int dtype, int rows, int V, int64_t ld, int rows_per_req,
                     const ss_req* req, const ss_aux* aux, void* ws, int32_t* out_ids) {
    Stage1Params p{};
    p.logits = logits;
    p.ld = ld;
    p.V = V;
    p.rows = rows;
    p.Zv = tiles_of(V, dtype);
    p.rows_per_req = rows_per_req;
    p.req = req;
    p.aux = aux_or_empty(aux);
    p.scratch = ws;
    p.out_ids = out_ids;
    p.aligned16 = aligned16(logits, dtype, ld);
    return p;
}

void launch_stage1(int dtype, const Stage1Params& p, hipStream_t s) {
    const int listed_wgs = (p.listed_rows + S1_WAVES - 1) / S1_WAVES;
    const dim3 grid((unsigned)(listed_wgs + p.rows * p.Zv)), block(S1_THREADS);
    if (dtype == SS_BF16) hipLaunchKernelGGL(stage1_kernel<SS_BF16>, grid, block, 0, s, p);
    else hipLaunchKernelGGL(stage1_kernel<SS_F32>, grid, block, 0, s, p);
}

// Rows whose lists are longer than LIST_SHORT are ranked by one more
// launch, issued only when the strides allow such lists.
void launch_listed_long(int dtype, const Stage1Params& p, hipStream_t s) {
    const bool long_prior = p.aux.prior_ids && p.aux.prior_cnt && p.aux.prior_stride > LIST_SHORT;
    const bool long_bias = p.aux.bias_ids && p.aux.bias_stride > LIST_SHORT;
    if (!(long_prior || long_bias) || p.listed_rows == 0) return;
    const dim3 grid((unsigned)p.listed_rows), block(LL_THREADS);
    if (dtype == SS_BF16) hipLaunchKernelGGL(listed_long_kernel<SS_BF16>, grid, block, 0, s, p);
    else hipLaunchKernelGGL(listed_long_kernel<SS_F32>, grid, block, 0, s, p);
}

template <int MODE>
void launch_stage2(int dtype, const Stage2Params& f, hipStream_t s) {
    const dim3 grid((unsigned)f.s1.rows), block(S2_THREADS);
    if (dtype == SS_BF16) hipLaunchKernelGGL((stage2_kernel<SS_BF16, MODE>), grid, block, 0, s, f);
    else hipLaunchKernelGGL((stage2_kernel<SS_F32, MODE>), grid, block, 0, s, f);
}

Stage2Params make_s2(const Stage1Params& s1, const ss_rng* rng, int mode, const WsLayout& L) {
    Stage2Params f{};
    f.s1 = s1;
    f.rng = rng;
    f.mode = mode;
    f.recs = L.recs;
    f.listed = L.listed;
    return f;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex noalloc_mu;
void* noalloc_ptr[NOALLOC_MAX_DEVICES];

int noalloc_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return SS_ERR_HIP;
    }
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return SS_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(noalloc_mu);
    if (!noalloc_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return SS_ERR_HIP;
        }
        noalloc_ptr[dev] = p;
    }
    *out = noalloc_ptr[dev];
    return SS_OK;
}

}  // namespace

namespace ssd {

__global__ void rng_advance_kernel(ss_rng* rng, uint64_t delta) {
    if (threadIdx.x == 0 && blockIdx.x == 0) rng->offset += delta;
}

// The epilogue's written functions, element by element over the arguments
// first + i (the same inline functions the sampling kernels call).
__global__ void spec_eval_kernel(int fn, uint32_t first, int64_t n, uint32_t c1, uint32_t c2, uint64_t seed,
                                 uint64_t offset, uint32_t* out) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const uint32_t a = first + (uint32_t)i;
        uint32_t r;
        switch (fn) {
        case SS_SPEC_EXP: r = fbits(exp_fixed_nonpos(bitsf(a))); break;
        case SS_SPEC_LOG: r = fbits(log_fixed(bitsf(a))); break;
        case SS_SPEC_LOG_NORMAL: r = fbits(log_fixed_normal(bitsf(a))); break;
        case SS_SPEC_GUMBEL_WORD: r = fbits(-log_fixed_normal(-log_fixed_normal(unit_open(a << 9)))); break;
        case SS_SPEC_PHILOX: r = philox_w0(seed, offset, a, c1, c2); break;
        default: r = fbits(gumbel_noise(seed, offset, a, c1, c2)); break;
        }
        out[i] = r;
    }
}

// A plain streaming read, the bandwidth reference of the measurements:
// 16-byte loads over the buffer (word i goes to workgroup (i mod
// 256*gridDim) / 256), four in flight per thread, with the streaming
// (nontemporal) policy of the logits loads; each workgroup xors what
// it read into out[blockIdx.x], so that no load can be dropped.
using sr_u32x4 = uint32_t __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void stream_read_kernel(const sr_u32x4* p, uint64_t n16, uint32_t* out) {
    __shared__ uint32_t s[4];
    const auto g = gmem(p);
    const uint64_t stride = (uint64_t)gridDim.x * 256u;
    uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const sr_u32x4 a = __builtin_nontemporal_load(g + i), b = __builtin_nontemporal_load(g + i + stride),
                      c = __builtin_nontemporal_load(g + i + 2 * stride), d = __builtin_nontemporal_load(g + i + 3 * stride);
        const sr_u32x4 x = a ^ b ^ c ^ d;
        acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
    }
    for (; i < n16; i += stride) {
        const sr_u32x4 a = __builtin_nontemporal_load(g + i);
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, WAVE);
    if ((threadIdx.x & (WAVE - 1)) == 0) s[threadIdx.x / WAVE] = acc;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

}  // namespace ssd

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

int ss_tile_size(int dtype) {
    if (dtype != SS_F32 && dtype != SS_BF16) return 0;
    return tile_of(dtype);
}

size_t ss_workspace_bytes(int rows, int V, int dtype) {
    if (rows < 0 || V < 1 || (dtype != SS_F32 && dtype != SS_BF16)) return 0;
    return ARRIVE_BYTES + scratch_bytes(rows, V, dtype) + listed_bytes(rows) + rec_bytes(rows) + RNG_SNAP_BYTES;
}

const char* ss_status_str(int status) {
    switch (status) {
        case SS_OK: return "ok";
        case SS_ERR_INVALID_ARG: return "invalid argument";
        case SS_ERR_UNSUPPORTED: return "unsupported dtype, size or gamma";
        case SS_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
        case SS_ERR_HIP: return "kernel launch failed";
        case SS_ERR_NOALLOC_LIMIT: return "call needs more workspace than the allocation-free entry point holds";
        default: return "unknown status";
    }
}

int ss_sample_step(const void* logits, int dtype, int B, int V, int64_t ld, const ss_req* req,
                   const ss_aux* aux, ss_rng* rng, uint64_t rng_advance, int32_t* out_tokens, int32_t* out_topk_ids,
                   float* out_probs, int32_t* out_kept, float* out_mass, int32_t* out_status, void* ws,
                   size_t ws_bytes, void* stream) {
    int rc = check_logits(logits, dtype, B, V, ld);
    if (rc) return rc;
    if ((rc = check_aux(aux, V))) return rc;
    if (B == 0) return SS_OK;
    if (!req || !rng || !out_tokens) return SS_ERR_INVALID_ARG;
    if ((rc = check_ws(ws, ws_bytes, ss_workspace_bytes(B, V, dtype)))) return rc;
    hipStream_t s = (hipStream_t)stream;
    const WsLayout W = ws_layout(ws, B, V, dtype);
    Stage1Params s1 = make_s1(logits, dtype, B, V, ld, 1, req, aux, W.scratch, nullptr);
    s1.listed = W.listed;
    s1.listed_rows = B;
    s1.rng = rng;
    s1.rng_snap = W.rng_snap;
    s1.rng_advance = rng_advance;
    launch_stage1(dtype, s1, s);
    launch_listed_long(dtype, s1, s);
    Stage2Params f = make_s2(s1, W.rng_snap, MODE_SAMPLE, W);
    f.tokens = out_tokens;
    f.topk_ids = out_topk_ids;
    f.probs = out_probs;
    f.kept = out_kept;
    f.mass = out_mass;
    f.status = out_status;
    launch_stage2<MODE_SAMPLE>(dtype, f, s);
    return launched();
}

int ss_sample_step_noalloc(const void* logits, int dtype, int B, int V, int64_t ld, const ss_req* req,
                           const ss_aux* aux, ss_rng* rng, uint64_t rng_advance, int32_t* out_tokens,
                           int32_t* out_topk_ids, float* out_probs, int32_t* out_kept, float* out_mass,
                           int32_t* out_status, void* stream) {
    // the same checks as ss_sample_step first, so that argument errors keep
    // their codes; then the size limit of the static workspace
    int rc = check_logits(logits, dtype, B, V, ld);
    if (rc) return rc;
    if ((rc = check_aux(aux, V))) return rc;
    if (B == 0) return SS_OK;
    if (!req || !rng || !out_tokens) return SS_ERR_INVALID_ARG;
    const size_t need = ss_workspace_bytes(B, V, dtype);
    if (need > (size_t)SS_NOALLOC_WS_BYTES) return SS_ERR_NOALLOC_LIMIT;
    void* ws = nullptr;
    if ((rc = noalloc_scratch(&ws))) return rc;
    // sampling reads nothing from the workspace that the same call did not
    // write first, so the array needs no clearing
    return ss_sample_step(logits, dtype, B, V, ld, req, aux, rng, rng_advance, out_tokens, out_topk_ids, out_probs,
                          out_kept, out_mass, out_status, ws, (size_t)SS_NOALLOC_WS_BYTES, stream);
}

int ss_verify_step(const void* target_logits, int dtype, int B, int gamma, int V, int64_t ld,
                   const ss_req* req, const ss_aux* aux, ss_rng* rng, uint64_t rng_advance, const int32_t* draft_ids,
                   const float* draft_probs, int32_t* out_tokens, int32_t* out_n_emit, int32_t* out_status,
                   void* ws, size_t ws_bytes, void* stream) {
    return ss_verify_step_var(target_logits, dtype, B, gamma, V, ld, req, aux, rng, rng_advance, nullptr, draft_ids,
                              draft_probs, out_tokens, out_n_emit, out_status, ws, ws_bytes, stream);
}

int ss_verify_step_var(const void* target_logits, int dtype, int B, int gamma, int V, int64_t ld,
                       const ss_req* req, const ss_aux* aux, ss_rng* rng, uint64_t rng_advance,
                       const int32_t* cu_num_draft, const int32_t* draft_ids, const float* draft_probs,
                       int32_t* out_tokens, int32_t* out_n_emit, int32_t* out_status,
                       void* ws, size_t ws_bytes, void* stream) {
    if (gamma < 1 || gamma > SS_GAMMA_MAX) return SS_ERR_UNSUPPORTED;
    if (B < 0 || (int64_t)B * (gamma + 1) > KERNEL_ROWS_MAX) return B < 0 ? SS_ERR_INVALID_ARG : SS_ERR_UNSUPPORTED;
    const int rows = B * (gamma + 1);
    int rc = check_logits(target_logits, dtype, rows, V, ld);
    if (rc) return rc;
    if ((rc = check_aux(aux, V))) return rc;
    if (B == 0) return SS_OK;
    if (!req || !rng || !draft_ids || !draft_probs || !out_tokens || !out_n_emit) return SS_ERR_INVALID_ARG;
    if ((rc = check_ws(ws, ws_bytes, ss_workspace_bytes(rows, V, dtype)))) return rc;
    hipStream_t s = (hipStream_t)stream;
    const WsLayout W = ws_layout(ws, rows, V, dtype);
    Stage1Params s1 = make_s1(target_logits, dtype, rows, V, ld, gamma + 1, req, aux, W.scratch, nullptr);
    s1.listed = W.listed;
    s1.listed_rows = rows;
    s1.cu_num_draft = cu_num_draft;
    s1.draft_ids = draft_ids;
    s1.rng = rng;
    s1.rng_snap = W.rng_snap;
    s1.rng_advance = rng_advance;
    if (B <= ARRIVE_REQUESTS_MAX) {   // Stage 2 decides and emits: its words start at zero
        s1.clear_words = (uint64_t*)W.arrive;
        s1.n_clear = B;
    }
    launch_stage1(dtype, s1, s);
    launch_listed_long(dtype, s1, s);
    Stage2Params f = make_s2(s1, W.rng_snap, MODE_VERIFY, W);
    f.gamma = gamma;
    f.draft_ids = draft_ids;
    f.draft_probs = draft_probs;
    f.cu_num_draft = cu_num_draft;
    f.v_tokens = out_tokens;
    f.v_n_emit = out_n_emit;
    f.v_status = out_status;
    if (B <= ARRIVE_REQUESTS_MAX) {   // Stage 2 decides and emits: two launches
        f.arrive = W.arrive;
        launch_stage2<MODE_VERIFY>(dtype, f, s);
        return launched();
    }
    launch_stage2<MODE_VERIFY>(dtype, f, s);
    hipLaunchKernelGGL(verify_kernel, dim3((unsigned)B), dim3(VF_THREADS), 0, s, f);
    return launched();
}

namespace {

int dense_tiles(int V) { return (V + DN_TILE - 1) / DN_TILE; }

// dense workspace: [tile keys][tile sums][draw keys][decisions][rng copy]
struct DenseWs {
    uint64_t* part_k;
    float* part_s;
    uint64_t* draw_k;
    DenseDec* dec;
    ss_rng* rng_snap;
    size_t bytes;
};
DenseWs dense_ws(void* ws, int B, int gamma, int V) {
    const size_t rz = (size_t)B * (gamma + 1) * dense_tiles(V), bz = (size_t)B * dense_tiles(V);
    DenseWs L;
    char* p = (char*)ws;
    size_t o = ARRIVE_BYTES;   // left alone: a workspace shared with the bounded path keeps its counters
    L.part_k = (uint64_t*)(p + o);
    o += align256(rz * sizeof(uint64_t));
    L.part_s = (float*)(p + o);
    o += align256(rz * sizeof(float));
    L.draw_k = (uint64_t*)(p + o);
    o += align256(bz * sizeof(uint64_t));
    L.dec = (DenseDec*)(p + o);
    o += align256((size_t)B * sizeof(DenseDec));
    L.rng_snap = (ss_rng*)(p + o);
    o += RNG_SNAP_BYTES;
    L.bytes = o;
    return L;
}

}  // namespace

size_t ss_verify_dense_workspace_bytes(int B, int gamma, int V) {
    if (B < 0 || gamma < 1 || gamma > SS_GAMMA_MAX || V < 1 || V > SS_V_MAX) return 0;
    return dense_ws(nullptr, B, gamma, V).bytes;
}

int ss_verify_step_dense(const void* target_logits, int dtype, int B, int gamma, int V, int64_t ld,
                         const ss_req* req, ss_rng* rng, uint64_t rng_advance, const int32_t* cu_num_draft,
                         const int32_t* draft_ids, const float* draft_probs, int32_t* out_tokens,
                         int32_t* out_n_emit, int32_t* out_status, void* ws, size_t ws_bytes, void* stream) {
    if (gamma < 1 || gamma > SS_GAMMA_MAX) return SS_ERR_UNSUPPORTED;
    if (B < 0 || (int64_t)B * (gamma + 1) > KERNEL_ROWS_MAX) return B < 0 ? SS_ERR_INVALID_ARG : SS_ERR_UNSUPPORTED;
    const int rows = B * (gamma + 1);
    int rc = check_logits(target_logits, dtype, rows, V, ld);
    if (rc) return rc;
    if ((int64_t)rows * dense_tiles(V) > 0x7FFFFFFFLL) return SS_ERR_UNSUPPORTED;
    if (B == 0) return SS_OK;
    if (!req || !rng || !draft_ids || !out_tokens || !out_n_emit) return SS_ERR_INVALID_ARG;
    if ((rc = check_ws(ws, ws_bytes, ss_verify_dense_workspace_bytes(B, gamma, V)))) return rc;
    const DenseWs L = dense_ws(ws, B, gamma, V);
    DenseParams D{};
    D.target = target_logits;
    D.dtype = dtype;
    D.B = B;
    D.G = gamma;
    D.V = V;
    D.Zt = dense_tiles(V);
    D.ld = ld;
    D.aligned16 = aligned16(target_logits, dtype, ld);
    D.req = req;
    D.rng = rng;
    D.rng_snap = L.rng_snap;
    D.rng_advance = rng_advance;
    D.cu_num_draft = cu_num_draft;
    D.draft_ids = draft_ids;
    D.draft_probs = draft_probs;
    D.part_k = L.part_k;
    D.part_s = L.part_s;
    D.draw_k = L.draw_k;
    D.dec = L.dec;
    D.out_tokens = out_tokens;
    D.out_n_emit = out_n_emit;
    D.out_status = out_status;
    hipStream_t s = (hipStream_t)stream;
    const dim3 blk(DN_THREADS);
    if (dtype == SS_BF16) {
        hipLaunchKernelGGL(dense_stats_kernel<SS_BF16>, dim3((unsigned)(rows * D.Zt)), blk, 0, s, D);
        hipLaunchKernelGGL(dense_draw_kernel<SS_BF16>, dim3((unsigned)(B * D.Zt)), blk, 0, s, D);
        hipLaunchKernelGGL(dense_finish_kernel<SS_BF16>, dim3((unsigned)B), dim3(WAVE), 0, s, D);
    } else {
        hipLaunchKernelGGL(dense_stats_kernel<SS_F32>, dim3((unsigned)(rows * D.Zt)), blk, 0, s, D);
        hipLaunchKernelGGL(dense_draw_kernel<SS_F32>, dim3((unsigned)(B * D.Zt)), blk, 0, s, D);
        hipLaunchKernelGGL(dense_finish_kernel<SS_F32>, dim3((unsigned)B), dim3(WAVE), 0, s, D);
    }
    return launched();
}

int ss_topk_step(const void* logits, int dtype, int B, int V, int64_t ld, int k, int32_t* out_ids,
                 float* out_vals, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_logits(logits, dtype, B, V, ld);
    if (rc) return rc;
    if (k < 1 || k > KMAX) return SS_ERR_UNSUPPORTED;
    if (B == 0) return SS_OK;
    if (!out_ids) return SS_ERR_INVALID_ARG;
    if ((rc = check_ws(ws, ws_bytes, ss_workspace_bytes(B, V, dtype)))) return rc;
    hipStream_t s = (hipStream_t)stream;
    const WsLayout W = ws_layout(ws, B, V, dtype);
    Stage1Params s1 = make_s1(logits, dtype, B, V, ld, 1, nullptr, nullptr, W.scratch, nullptr);
    launch_stage1(dtype, s1, s);
    Stage2Params f = make_s2(s1, nullptr, MODE_TOPK, W);
    f.topk_k = k;
    f.topk_ids = out_ids;
    f.topk_vals = out_vals;
    launch_stage2<MODE_TOPK>(dtype, f, s);
    return launched();
}

int ss_topk_step_radix(const void* logits, int dtype, int B, int V, int64_t ld, int k, int32_t* out_ids,
                       float* out_vals, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_logits(logits, dtype, B, V, ld);
    if (rc) return rc;
    if (k < 1 || k > KMAX) return SS_ERR_UNSUPPORTED;
    if (B == 0) return SS_OK;
    if (!out_ids) return SS_ERR_INVALID_ARG;
    if ((rc = check_ws(ws, ws_bytes, ss_workspace_bytes(B, V, dtype)))) return rc;
    hipStream_t s = (hipStream_t)stream;
    const WsLayout W = ws_layout(ws, B, V, dtype);
    Stage1Params s1 = make_s1(logits, dtype, B, V, ld, 1, nullptr, nullptr, W.scratch, nullptr);
    const dim3 grid((unsigned)(B * s1.Zv)), block(S1_THREADS);
    if (dtype == SS_BF16) hipLaunchKernelGGL(stage1_radix_kernel<SS_BF16>, grid, block, 0, s, s1);
    else hipLaunchKernelGGL(stage1_radix_kernel<SS_F32>, grid, block, 0, s, s1);
    Stage2Params f = make_s2(s1, nullptr, MODE_TOPK, W);
    f.topk_k = k;
    f.topk_ids = out_ids;
    f.topk_vals = out_vals;
    launch_stage2<MODE_TOPK>(dtype, f, s);
    return launched();
}

int ss_topk_single_pass(const void* logits, int dtype, int B, int V, int64_t ld, int k, int32_t* out_ids,
                        float* out_vals, void* stream) {
    int rc = check_logits(logits, dtype, B, V, ld);
    if (rc) return rc;
    if (k < 1 || k > KMAX) return SS_ERR_UNSUPPORTED;
    if (B == 0) return SS_OK;
    if (!out_ids) return SS_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    const int al = aligned16(logits, dtype, ld);
    if (dtype == SS_BF16)
        hipLaunchKernelGGL(topk_radix_row_kernel<SS_BF16>, dim3((unsigned)B), dim3(RR_THREADS), 0, s, logits, V, ld,
                           al, k, out_ids, out_vals);
    else
        hipLaunchKernelGGL(topk_radix_row_kernel<SS_F32>, dim3((unsigned)B), dim3(RR_THREADS), 0, s, logits, V, ld,
                           al, k, out_ids, out_vals);
    return launched();
}

int ss_tile_topk(const void* logits, int dtype, int rows, int V, int64_t ld, int rows_per_req, const ss_req* req,
                 const ss_aux* aux, int32_t* out_ids, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_logits(logits, dtype, rows, V, ld);
    if (rc) return rc;
    if ((rc = check_aux(aux, V))) return rc;
    if (rows_per_req < 1) return SS_ERR_INVALID_ARG;
    if (rows == 0) return SS_OK;
    if ((rc = check_ws(ws, ws_bytes, ss_workspace_bytes(rows, V, dtype)))) return rc;
    hipStream_t s = (hipStream_t)stream;
    const WsLayout W = ws_layout(ws, rows, V, dtype);
    Stage1Params s1 = make_s1(logits, dtype, rows, V, ld, rows_per_req, req, aux, W.scratch, out_ids);
    if (req) {   // the steps' own Stage-1 launch: the rows' listed tokens are ranked too
        s1.listed = W.listed;
        s1.listed_rows = rows;
    }
    launch_stage1(dtype, s1, s);
    return launched();
}

int ss_stream_read(const void* p, size_t bytes, int nblocks, uint32_t* out, void* stream) {
    if (nblocks < 1 || nblocks > (1 << 20)) return SS_ERR_UNSUPPORTED;
    if (!out || (bytes && !p) || ((uintptr_t)p & 15u) || (bytes & 15u)) return SS_ERR_INVALID_ARG;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)nblocks), dim3(256), 0, (hipStream_t)stream,
                       (const sr_u32x4*)p, (uint64_t)(bytes / 16), out);
    return launched();
}

int ss_spec_eval(int fn, uint32_t first, int64_t n, uint32_t c1, uint32_t c2, uint64_t seed, uint64_t offset,
                 uint32_t* out, void* stream) {
    if (fn < SS_SPEC_EXP || fn > SS_SPEC_GUMBEL || n < 0 || n > ((int64_t)1 << 32)) return SS_ERR_INVALID_ARG;
    if (n == 0) return SS_OK;
    if (!out) return SS_ERR_INVALID_ARG;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(spec_eval_kernel, dim3((unsigned)(blocks < 16384 ? blocks : 16384)), dim3(256), 0,
                       (hipStream_t)stream, fn, first, n, c1, c2, seed, offset, out);
    return launched();
}

int ss_rng_advance(ss_rng* rng, uint64_t delta, void* stream) {
    if (!rng) return SS_ERR_INVALID_ARG;
    hipLaunchKernelGGL(rng_advance_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, rng, delta);
    return launched();
}

}  // extern "C"

namespace {

// probe columns: whole fp32 tiles, at least LM_PROBE_MIN and V / 16, so
// that about (V / P - 1) * 128 <= 15 * 128 tokens per row pass its
// threshold
int lm_probe_cols(int V) {
    const int64_t t = S1Traits<SS_F32>::BN;
    int64_t p = ((int64_t)V / 16 + t - 1) / t * t;
    if (p < LM_PROBE_MIN) p = LM_PROBE_MIN;
    return (int)(p < V ? p : V);
}

// LM-head workspace: [Stage-1 workspace of the probe][probe logits
// B x P fp32][candidates B x LM_CAP][counts B][logits of the other columns
// B x (V - P) fp32, written only for rows whose candidates overflowed]
struct LmWs {
    void* std_ws;
    size_t std_bytes;
    float* probe;
    uint64_t* cand;
    int32_t* cnt;
    float* rest;
    size_t bytes;
};
LmWs lm_ws(void* ws, int B, int V) {
    const int P = lm_probe_cols(V);
    LmWs L;
    char* p = (char*)ws;
    size_t o = 0;
    L.std_ws = p;
    L.std_bytes = ss_workspace_bytes(B, P, SS_F32);
    o += align256(L.std_bytes);
    L.probe = (float*)(p + o);
    o += align256((size_t)B * P * sizeof(float));
    L.cand = (uint64_t*)(p + o);
    o += align256((size_t)B * LM_CAP * sizeof(uint64_t));
    L.cnt = (int32_t*)(p + o);
    o += align256((size_t)B * sizeof(int32_t));
    L.rest = (float*)(p + o);
    o += align256((size_t)B * (V - P) * sizeof(float));
    L.bytes = o;
    return L;
}

int check_lmhead(const void* hidden, int64_t ldh, const void* weight, int64_t ldw, int B, int D, int V) {
    if (B < 0 || V < 1 || D < 1 || ldh < D || ldw < D) return SS_ERR_INVALID_ARG;
    if (V > SS_V_MAX || D % 128 != 0 || D > (1 << 16) || (ldh % 8) || (ldw % 8)) return SS_ERR_UNSUPPORTED;
    if (B > 0 && (!hidden || !weight)) return SS_ERR_INVALID_ARG;
    if (((uintptr_t)hidden & 15u) || ((uintptr_t)weight & 15u)) return SS_ERR_UNSUPPORTED;
    return SS_OK;
}

template <int MODE, int WM, int WNW, int WN, int KB, bool SPLIT, bool NTW>
void lm_launch(LmParams p, hipStream_t s) {
    constexpr int MT = 64 * WM, NT = WNW * 32 * WN;
    constexpr int threads = (WM * WNW + (SPLIT ? 4 : 0)) * WAVE;
    const int ncols = p.col_end - p.col_begin;
    p.ncol_tiles = (ncols + NT - 1) / NT;
    p.nrow_tiles = (p.B + MT - 1) / MT;
    const int64_t blocks = p.nrow_tiles == 1 ? p.ncol_tiles
                                             : (int64_t)(p.ncol_tiles + 7) / 8 * 8 * p.nrow_tiles;
    hipLaunchKernelGGL((lmhead_gemm_kernel<MODE, WM, WNW, WN, KB, SPLIT, NTW>), dim3((unsigned)blocks),
                       dim3(threads), 0, s, p);
}

// launch shapes (four multiplying waves each; rows x columns per
// workgroup): B <= 64 one row tile of 64 rows (waves side by side);
// B <= 128 one row tile of 128 (2 x 2 waves); larger B row tiles of 256
// (waves stacked, 128 columns), so that each weight column is read by
// fewer workgroups, with four more waves issuing the loads.  A launch with
// one row tile reads the weights with the nt policy (B=64, D=4096,
// V=2^17: logits 204 -> 174 us, fused step 243 -> 215 us).  Measured at
// B=256, D=4096, V=2^18 (logits / fused step, one run): 128-row tiles
// 677 / 797 us, 256-row tiles with the loading waves and the nt policy
// 611 / 749 us.  The probe covers few columns, so it uses tiles of 128
// rows by 64 columns (rows past B repeat the last one) and long k stages:
// twice the workgroups of 64 x 128 or 128 x 128 tiles, and each runs alone
// on a CU waiting on memory (fused step at B=128: 498 -> 472 us; B=64 and
// B=256 unchanged; with the nt policy the probe is slower).
template <int MODE>
void lm_launch_shape(LmParams p, bool probe, hipStream_t s) {
    if (probe) lm_launch<MODE, 2, 2, 1, 128, false, false>(p, s);
    else if (p.B <= 64) lm_launch<MODE, 1, 4, 2, 64, false, true>(p, s);
    else if (p.B <= 128) lm_launch<MODE, 2, 2, 4, 64, false, true>(p, s);
    else if (p.B <= 256) lm_launch<MODE, 4, 1, 4, 64, true, true>(p, s);
    else lm_launch<MODE, 4, 1, 4, 64, true, false>(p, s);
}

void launch_lm_gemm(int mode, LmParams p, bool probe, hipStream_t s) {
    const int ncols = p.col_end - p.col_begin;
    if (ncols <= 0 || p.B == 0) return;
    if (mode == LM_STORE) lm_launch_shape<LM_STORE>(p, probe, s);
    else if (mode == LM_THRESH) lm_launch_shape<LM_THRESH>(p, probe, s);
    else lm_launch_shape<LM_REDO>(p, probe, s);
}

}  // namespace

extern "C" {

size_t ss_lmhead_workspace_bytes(int B, int V) {
    if (B < 0 || V < 1 || V > SS_V_MAX) return 0;
    return lm_ws(nullptr, B, V).bytes;
}

int ss_lmhead_logits(const void* hidden, int64_t ldh, const void* weight, int64_t ldw, int B, int D, int V,
                     float* out_logits, int64_t ldo, void* stream) {
    int rc = check_lmhead(hidden, ldh, weight, ldw, B, D, V);
    if (rc) return rc;
    if (ldo < V) return SS_ERR_INVALID_ARG;
    if (B == 0) return SS_OK;
    if (!out_logits) return SS_ERR_INVALID_ARG;
    LmParams p{};
    p.H = (const uint16_t*)hidden;
    p.ldh = ldh;
    p.W = (const uint16_t*)weight;
    p.ldw = ldw;
    p.B = B;
    p.D = D;
    p.V = V;
    p.col_begin = 0;
    p.col_end = V;
    p.out = out_logits;
    p.ldo = ldo;
    launch_lm_gemm(LM_STORE, p, false, (hipStream_t)stream);
    return launched();
}

int ss_lmhead_sample_step(const void* hidden, int64_t ldh, const void* weight, int64_t ldw, int B, int D, int V,
                          const ss_req* req, ss_rng* rng, uint64_t rng_advance, int32_t* out_tokens,
                          int32_t* out_topk_ids, float* out_probs, int32_t* out_kept, float* out_mass,
                          int32_t* out_status, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_lmhead(hidden, ldh, weight, ldw, B, D, V);
    if (rc) return rc;
    if ((int64_t)B * tiles_of(lm_probe_cols(V), SS_F32) > 0x7FFFFFFFLL) return SS_ERR_UNSUPPORTED;
    if (B == 0) return SS_OK;
    if (!req || !rng || !out_tokens) return SS_ERR_INVALID_ARG;
    if ((rc = check_ws(ws, ws_bytes, ss_lmhead_workspace_bytes(B, V)))) return rc;
    hipStream_t s = (hipStream_t)stream;
    const int P = lm_probe_cols(V);
    const LmWs L = lm_ws(ws, B, V);
    // 1. the probe columns' logits
    LmParams g{};
    g.H = (const uint16_t*)hidden;
    g.ldh = ldh;
    g.W = (const uint16_t*)weight;
    g.ldw = ldw;
    g.B = B;
    g.D = D;
    g.V = V;
    g.col_begin = 0;
    g.col_end = P;
    g.out = L.probe;
    g.ldo = P;
    launch_lm_gemm(LM_STORE, g, true, s);
    // 2. their 128 best per row and probe tile; the step's generator copy;
    //    the candidate counts cleared
    const WsLayout W = ws_layout(L.std_ws, B, P, SS_F32);
    Stage1Params s1 = make_s1(L.probe, SS_F32, B, P, P, 1, req, nullptr, W.scratch, nullptr);
    s1.rng = rng;
    s1.rng_snap = W.rng_snap;
    s1.rng_advance = rng_advance;
    s1.clear_words = (uint64_t*)L.cnt;
    s1.n_clear = (B + 1) / 2;
    launch_stage1(SS_F32, s1, s);
    // 3. the other columns: every token above the probe's 128th
    g.col_begin = P;
    g.col_end = V;
    g.out = nullptr;
    g.probe_keys = (const uint64_t*)W.scratch;
    g.Zp = tiles_of(P, SS_F32);
    g.cand = L.cand;
    g.cnt = L.cnt;
    launch_lm_gemm(LM_THRESH, g, false, s);
    // 4. rows whose candidates overflowed: their other columns stored
    g.probe_keys = nullptr;
    g.cand = nullptr;
    g.out = L.rest;
    g.ldo = V - P;
    launch_lm_gemm(LM_REDO, g, false, s);
    // 5. merge and sample
    LmStage2Params q{};
    q.f = make_s2(s1, W.rng_snap, MODE_SAMPLE, W);
    q.f.s1.V = V;
    q.f.tokens = out_tokens;
    q.f.topk_ids = out_topk_ids;
    q.f.probs = out_probs;
    q.f.kept = out_kept;
    q.f.mass = out_mass;
    q.f.status = out_status;
    q.probe_keys = (const uint64_t*)W.scratch;
    q.Zp = tiles_of(P, SS_F32);
    q.cand = L.cand;
    q.cnt = L.cnt;
    q.probe = L.probe;
    q.rest = L.rest;
    q.P = P;
    hipLaunchKernelGGL(lmhead_stage2_kernel, dim3((unsigned)B), dim3(S2_THREADS), 0, s, q);
    return launched();
}

}  // extern "C"
