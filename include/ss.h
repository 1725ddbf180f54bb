/*
 * ss.h - C ABI of libss, the MI355X (gfx950) fused LLM sampling and
 * speculative-verification library.
 *
 * What the library computes is the sampling pipeline of "SonicSampler:
 * Unified Tile-Aware Kernels for LLM Sampling and Speculative Verification"
 * (arXiv 2607.20475):
 *   - per-request logits processing (section 3.1 "Logits processing"):
 *     grammar bitmask, repetition penalty, frequency and presence
 *     penalties, logit bias, temperature;
 *   - a two-stage tile-aware top-k with a bounded candidate set k = 128
 *     (section 3.2 "Workload-aware execution model", section 3.3, Fig. 1);
 *   - top-p / min-p truncation (section 3.1 "Probability truncation", the
 *     min-p condition evaluated without a softmax);
 *   - Gumbel-max token selection (section 3.1 "Sampling");
 *   - speculative rejection-sampling verification with residual
 *     max(0, p - q) resampling (section 3.1 "Speculative verification").
 * The notes page "Decoding and sampling" (sections "Temperature", "Top-k",
 * "Top-p", "Min-p", "Combination order", "Rejection Sampler") supplies the
 * set definitions and the rejection-sampling identities.
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless marked "host".  The caller owns
 *     every buffer, the workspace included.  The library never allocates,
 *     frees, or synchronises; all work is queued on `stream` (a
 *     hipStream_t passed as void*, NULL = the default stream).  Every
 *     launch uses a grid fixed by the shapes, and the random seed/offset
 *     are read from device memory, so a call can be captured in a hipGraph
 *     and replayed.
 *   - Return value: SS_OK, or a negative ss_status for problems found on
 *     the host before anything is launched (then nothing is launched), or
 *     SS_ERR_HIP when a launch failed.  Data-dependent problems never stop
 *     the call; they are reported per row in `out_status` (SS_ROW_*).
 *   - Logits: row-major, `rows` rows of `V` values with a row stride of
 *     `ld` elements (ld >= V), fp32 or bf16 (raw 16-bit patterns).
 *   - Tokens are int32 ids in [0, V); -1 means "no token".
 *   - Results are deterministic functions of the inputs and of
 *     (seed, offset); they do not depend on launch order or timing.
 */
#ifndef SS_H
#define SS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SS_KMAX 128        /* bounded candidate set (SonicSampler section 3.3) */
#define SS_GAMMA_MAX 16    /* largest number of draft tokens per request */
#define SS_V_MAX (1 << 24) /* largest vocabulary */
#define SS_PRIOR_MAX 4096  /* longest prior (penalty history) list per request */
#define SS_BIAS_MAX 1024   /* longest logit-bias list per request */
/* size of the static workspace behind ss_sample_step_noalloc, per GPU */
#define SS_NOALLOC_WS_BYTES (16u << 20)

typedef enum {
    SS_OK = 0,
    SS_ERR_INVALID_ARG = -1, /* null pointer, bad size, bad stride */
    SS_ERR_UNSUPPORTED = -2, /* dtype, V or gamma outside what is supported */
    SS_ERR_WORKSPACE = -3,   /* workspace missing, too small or misaligned */
    SS_ERR_HIP = -4,         /* a kernel launch failed */
    SS_ERR_NOALLOC_LIMIT = -5 /* ss_sample_step_noalloc: the call needs more than
                                 SS_NOALLOC_WS_BYTES of workspace */
} ss_status;

typedef enum { SS_F32 = 0, SS_BF16 = 1 } ss_dtype;

/* Per-row status written to out_status. */
enum {
    SS_ROW_OK = 0,
    SS_ROW_ALL_MASKED = 1,   /* every candidate is -inf: token -1 */
    SS_ROW_INVALID = 2,      /* a request field is out of range: token -1 */
    SS_ROW_TOPK_CLAMPED = 3  /* top_k > 128 was clamped to 128; token valid */
};

/* Per-request bit-level indicators (SonicSampler section 1: "compact
 * bit-level indicators" select each request's behaviour). */
enum {
    SS_GREEDY = 1u << 0,    /* argmax of the processed logits */
    SS_GRAMMAR = 1u << 1,   /* apply the row's grammar bitmask */
    SS_REP = 1u << 2,       /* repetition penalty over the prior list */
    SS_FREQPRES = 1u << 3,  /* frequency and presence penalties over the prior list */
    SS_BIAS = 1u << 4,      /* additive logit bias list */
    SS_TOPK = 1u << 5,      /* keep the top_k best candidates */
    SS_TOPP = 1u << 6,      /* nucleus truncation at top_p */
    SS_MINP = 1u << 7,      /* keep p_i >= min_p * p_max */
    /* verification only: target position j's penalty history (SS_REP,
     * SS_FREQPRES) is the prior list plus the request's drafts
     * d_0..d_{j-1}, each adding one occurrence to the first prior entry of
     * its id with a count >= 1, else to an entry appended for it (the
     * decoding notes' penalties act on every token generated so far) */
    SS_DRAFT_HIST = 1u << 8
};

/* One request, 32 bytes, in device memory (so a captured graph can be
 * replayed with new settings).  Field semantics:
 *   flags        SS_* bits above.
 *   top_k        with SS_TOPK: 1 means greedy, 2..128 bound the candidates,
 *                > 128 is clamped (SS_ROW_TOPK_CLAMPED), 0 is invalid.
 *                Without SS_TOPK the bound is 128.
 *   temperature  stochastic rows need a finite T > 0; T <= 0 means greedy;
 *                NaN or +inf makes the row invalid (unless SS_GREEDY).
 *   n_prior      entries of the row's prior list used (<= prior_stride and
 *                <= SS_PRIOR_MAX, else the row is invalid): the penalty
 *                history, every distinct token generated so far with its
 *                count.
 *   n_bias       entries of the row's bias list used (<= bias_stride and
 *                <= SS_BIAS_MAX, else the row is invalid).
 *   top_p        with SS_TOPP: in (0, 1]; 1 keeps every candidate.
 *   min_p        with SS_MINP: in [0, 1]; 0 keeps every candidate.
 *   rep_penalty  with SS_REP: finite, > 0 (theta).
 *   freq_penalty, pres_penalty  with SS_FREQPRES: finite. */
typedef struct ss_req {
    uint16_t flags;
    uint16_t top_k;
    float temperature;
    uint16_t n_prior;
    uint16_t n_bias;
    float top_p;
    float min_p;
    float rep_penalty;
    float freq_penalty;
    float pres_penalty;
} ss_req;

/* Philox seed and offset, in DEVICE memory; the kernels read them at run
 * time, so a captured graph draws new noise after ss_rng_advance, or on
 * every replay when the step advances the offset itself (rng_advance). */
typedef struct ss_rng {
    uint64_t seed;
    uint64_t offset;
} ss_rng;

/* Side arrays, passed as a HOST struct of device pointers.  Row r of a
 * call uses list row `r` (sample/tile calls) or `r / (gamma+1)` (verify,
 * i.e. the request), and bitmask row `r`.
 *   prior_ids/prior_cnt  [*, prior_stride] int32: token id and its count in
 *                        the request's history; entries with count < 1 or an
 *                        id outside [0, V) are ignored.
 *   bias_ids/bias_val    [*, bias_stride]: token id and additive bias
 *                        (finite); ids outside [0, V) are ignored.
 *   bitmask              [rows, bitmask_stride] uint32, bitmask_stride >=
 *                        ceil(V/32): token i is allowed iff bit (i & 31) of
 *                        word (i >> 5) is 1.
 * Any pointer may be NULL when no row uses it; a row whose flags need a
 * NULL array is SS_ROW_INVALID.
 * Processing order per token (SonicSampler section 3.1): mask (-inf), then
 * every prior entry in list order z = z>0 ? z/theta : z*theta (SS_REP), then
 * every prior entry z = z - (count*freq + presence) (SS_FREQPRES), then
 * every bias entry z = z + bias (SS_BIAS); finally NaN -> -inf,
 * +inf -> FLT_MAX, -0 -> +0. */
typedef struct ss_aux {
    const int32_t* prior_ids;
    const int32_t* prior_cnt;
    int32_t prior_stride;
    const int32_t* bias_ids;
    const float* bias_val;
    int32_t bias_stride;
    const uint32_t* bitmask;
    int64_t bitmask_stride;
} ss_aux;

/* Bytes of workspace a call over `rows` logits rows of width V needs (rows
 * = B for sampling and top-k, B*(gamma+1) for verification).  Pure host
 * function; the workspace must be 256-byte aligned and needs no
 * initialisation (its first 4096 bytes hold verification's per-request
 * decision words, which each verification step clears in its first launch).
 * One workspace can serve any sequence of calls and graph replays; calls
 * that share a workspace must not overlap in time. */
size_t ss_workspace_bytes(int rows, int V, int dtype);

/* Vocabulary tile width used for `dtype` (B_N of the two-stage top-k). */
int ss_tile_size(int dtype);

/* Single-step sampling (SonicSampler "single-step mode").
 * For every row b of the B x V logits:
 *   z   = processed logits (see ss_aux);
 *   K   = min(top_k if SS_TOPK else 128, 128, V) best tokens by
 *         (z descending, token id ascending);
 *   greedy rows (SS_GREEDY, T <= 0 or top_k == 1): token = best id;
 *   otherwise v_k = z_k / T computed as z_k * (1/T) and clamped to the
 *   finite range, e_k = exp(v_k - v_1) (fixed polynomial exp), Z = e_1 +
 *   ... + e_K summed left to right, E_k the running sums; top-p keeps rank
 *   k while E_{k-1} < top_p * Z, min-p keeps v_k - v_1 >= ln(min_p); the
 *   token is the argmax over the kept ranks of v_k + g(id_k), with Gumbel
 *   noise g = -ln(-ln u) from Philox4x32-10 (counter = {id, b, 0,
 *   offset_lo}, key = {seed_lo, seed_hi ^ offset_hi}, u = ((w0 >> 9) +
 *   1/2) * 2^-23); ties go to the lower id.
 * Outputs (all optional except out_tokens):
 *   out_tokens [B] int32, out_topk_ids [B,128] int32 (the K candidates, -1
 *   after), out_probs [B,128] float (e_k / Z; greedy rows 1,0,...),
 *   out_kept [B] int32 (kept count), out_mass [B] float (kept mass / Z),
 *   out_status [B] int32 (SS_ROW_*).
 * rng_advance: the step copies *rng into its workspace in its first launch
 * and then adds rng_advance to rng->offset on the device (0 leaves *rng
 * untouched); its own draws use the copied offset.  A decode loop or a
 * captured graph thus needs no separate ss_rng_advance. */
int ss_sample_step(const void* logits, int dtype, int B, int V, int64_t ld,
                   const ss_req* req, const ss_aux* aux, ss_rng* rng, uint64_t rng_advance,
                   int32_t* out_tokens, int32_t* out_topk_ids, float* out_probs,
                   int32_t* out_kept, float* out_mass, int32_t* out_status,
                   void* ws, size_t ws_bytes, void* stream);

/* ss_sample_step for callers that cannot allocate device memory (code
 * under hipGraph capture that must not call hipMalloc, tight serving loops,
 * harnesses that forbid allocation): the same arguments, computation,
 * outputs and errors, without the workspace arguments.  Its workspace is a
 * device array inside the library, SS_NOALLOC_WS_BYTES (16 MiB) on each GPU
 * it runs on, held until the process ends; its address on the current
 * device is looked up on the first call there.  A call whose
 * ss_workspace_bytes(B, V, dtype) exceeds SS_NOALLOC_WS_BYTES returns
 * SS_ERR_NOALLOC_LIMIT before anything is launched (e.g. B = 256 at V =
 * 2^18 bf16 needs about 1.7 MiB; B = 2048 at V = 2^18 fp32 is too large).
 * The call allocates nothing and launches the same kernels as
 * ss_sample_step.  Every call on one GPU shares that GPU's array, which
 * keeps the last call's contents (a call reads only what it wrote itself,
 * so nothing needs clearing): calls that overlap in time on one GPU, e.g.
 * on two streams, race and give wrong results; serialise them.  The
 * current device must be the device of `stream`. */
int ss_sample_step_noalloc(const void* logits, int dtype, int B, int V, int64_t ld,
                           const ss_req* req, const ss_aux* aux, ss_rng* rng, uint64_t rng_advance,
                           int32_t* out_tokens, int32_t* out_topk_ids, float* out_probs,
                           int32_t* out_kept, float* out_mass, int32_t* out_status, void* stream);

/* Speculative verification of `gamma` draft tokens per request
 * (SonicSampler "multi-step mode").  target_logits has B*(gamma+1) rows;
 * row b*(gamma+1)+j is the target distribution for position j of request b
 * (position gamma gives the bonus token).  req[b] and the prior/bias list
 * row b belong to request b; bitmask rows follow the target rows.
 * p_j is the request's truncated, renormalised target distribution at
 * position j (ss_sample_step's kept set, p = e_k / E_n).  draft_ids [B,
 * gamma] int32 and draft_probs [B, gamma, V] fp32 (q_j, read only at the
 * draft token and at the kept candidates).
 * Stochastic requests, for j = 0..gamma-1: accept d_j iff q_j(d_j) > 0 and
 * u_j * q_j(d_j) <= p_j(d_j) with u_j from Philox counter {0, b, (1<<24)|j,
 * offset_lo}; at the first rejection emit argmax over kept ranks with
 * rho_k = max(0, p_j - q_j) > 0 of ln(rho_k) + g (counter {id, b,
 * (2<<24)|j}) - or, if every rho_k is 0, the Gumbel-max draw from p_j with
 * that counter - and stop.  If all are accepted emit the Gumbel-max draw
 * from position gamma (counter {id, b, gamma}).  Greedy requests accept
 * d_j iff it equals the best id of row j, emit the best id at the first
 * mismatch and stop, and emit the best id of row gamma when all match.
 * Outputs: out_tokens [B, gamma+1] (-1 after the emitted ones), out_n_emit
 * [B], out_status [B] (optional; SS_ROW_ALL_MASKED when a target row that
 * is reached has no finite candidate).  rng_advance as for
 * ss_sample_step. */
int ss_verify_step(const void* target_logits, int dtype, int B, int gamma, int V, int64_t ld,
                   const ss_req* req, const ss_aux* aux, ss_rng* rng, uint64_t rng_advance,
                   const int32_t* draft_ids, const float* draft_probs,
                   int32_t* out_tokens, int32_t* out_n_emit, int32_t* out_status,
                   void* ws, size_t ws_bytes, void* stream);

/* ss_verify_step with a per-request number of drafts (the decoding notes,
 * "Rejection Sampler": the verification kernel takes each request's draft
 * range from cumulative offsets, cu_num_draft_tokens).  cu_num_draft
 * [B] int32 in device memory holds inclusive cumulative counts, so request
 * b has n_b = cu[b] - cu[b-1] (cu[-1] = 0) drafts.  The tensors keep the
 * gamma-wide layout of ss_verify_step (gamma is the largest count): request
 * b's drafts are draft_ids[b, 0..n_b-1] and draft_probs[b, 0..n_b-1], its
 * target rows are b*(gamma+1) + 0..n_b, and row n_b gives its bonus token;
 * rows, drafts and probabilities past n_b are not used (they are still read
 * by the tile stage, so keep them finite or masked).  A count outside
 * [0, gamma] makes the request SS_ROW_INVALID (no token emitted).  The
 * counts are read on the device, so the call stays graph-capturable.
 * cu_num_draft = NULL is ss_verify_step. */
int ss_verify_step_var(const void* target_logits, int dtype, int B, int gamma, int V, int64_t ld,
                       const ss_req* req, const ss_aux* aux, ss_rng* rng, uint64_t rng_advance,
                       const int32_t* cu_num_draft, const int32_t* draft_ids, const float* draft_probs,
                       int32_t* out_tokens, int32_t* out_n_emit, int32_t* out_status,
                       void* ws, size_t ws_bytes, void* stream);

/* Dense verification (decoding notes, "Rejection Sampler": the rejection
 * and recovery kernels read whole target and draft probability rows).
 * p_j is the softmax of v = z/T over the WHOLE vocabulary: z the canonical
 * target logits, no candidate bound and no truncation (top_k, top_p, min_p
 * do not apply); T as in ss_req (SS_GREEDY or T <= 0: greedy).  A request
 * that asks for a grammar mask, penalties, bias or SS_DRAFT_HIST is
 * SS_ROW_INVALID here (no logits processing in this variant).
 *   target_logits [B*(gamma+1), ld] as in ss_verify_step.
 *   draft_probs   [B, gamma, V] fp32 rows, or NULL: no draft probabilities
 *                 (q counts as 1 at the draft token; a rejection draws from
 *                 p with the draft token left out).
 *   cu_num_draft  NULL or the inclusive cumulative draft counts, as in
 *                 ss_verify_step_var.
 * Draft d_j is accepted when q_j(d_j) > 0 and u_j q_j(d_j) <= p_j(d_j); at
 * the first rejection the token is the Gumbel-max of ln max(0, p_j - q_j)
 * over the vocabulary (p where q >= p everywhere); when every draft is
 * accepted the bonus is the Gumbel-max of v over row n_b.  Greedy requests
 * accept a draft equal to the row's best id.  Outputs, statuses, noise
 * counters, rng and rng_advance as in ss_verify_step.  ws: at least
 * ss_verify_dense_workspace_bytes(B, gamma, V) bytes, 256-byte aligned;
 * its first 4096 bytes are not touched (they may hold the counters of a
 * workspace shared with ss_workspace_bytes users). */
size_t ss_verify_dense_workspace_bytes(int B, int gamma, int V);
int ss_verify_step_dense(const void* target_logits, int dtype, int B, int gamma, int V, int64_t ld,
                         const ss_req* req, ss_rng* rng, uint64_t rng_advance,
                         const int32_t* cu_num_draft, const int32_t* draft_ids, const float* draft_probs,
                         int32_t* out_tokens, int32_t* out_n_emit, int32_t* out_status,
                         void* ws, size_t ws_bytes, void* stream);

/* Two-stage top-k of raw logits (no processing beyond NaN -> -inf, +inf ->
 * FLT_MAX, -0 -> +0): out_ids [B, k] in order (value descending, id
 * ascending) and out_vals [B, k] (optional) their values; positions past V
 * hold -1 / -inf.  1 <= k <= 128. */
int ss_topk_step(const void* logits, int dtype, int B, int V, int64_t ld, int k,
                 int32_t* out_ids, float* out_vals, void* ws, size_t ws_bytes, void* stream);

/* The same result as ss_topk_step (same arguments, workspace and errors),
 * with the tile stage selecting by the adaptive radix-bitonic strategy of
 * the SonicSampler paper (Fig. 1, right panel): a 6-bit screen of the
 * 16-bit order key, then either the bitonic select of the survivors at once
 * or a radix pass over the next 10 bits first (more than 256 elements tied
 * at 16-bit precision take the threshold path, so the result is exact for
 * every input).  For comparison with ss_topk_step's threshold select. */
int ss_topk_step_radix(const void* logits, int dtype, int B, int V, int64_t ld, int k,
                       int32_t* out_ids, float* out_vals, void* ws, size_t ws_bytes, void* stream);

/* The same result as ss_topk_step from one program per row (the design the
 * two-stage method replaces, SonicSampler section 3.2; radix select as
 * section 3.1 "Top-k selection primitives" describes it): one workgroup per
 * row streams the whole row once per pass, each pass histograms the next
 * 8-bit digit of the order key among the elements matching the digits of
 * the k-th key found so far, and once at most 1024 elements lie at or above
 * that prefix one more pass gathers them for an exact sort; ties at a fully
 * resolved k-th value are settled by a radix select over the token index
 * (lower id first).  Needs no workspace; errors as ss_topk_step. */
int ss_topk_single_pass(const void* logits, int dtype, int B, int V, int64_t ld, int k,
                        int32_t* out_ids, float* out_vals, void* stream);

/* Stage 1 alone (diagnostic and timing): fills the workspace with every
 * tile's 128 best tokens, and when out_ids is not NULL also writes them as
 * token ids, [rows, ceil(V/tile), 128] int32 (-1 where a tile has fewer).
 * Tokens named by an active penalty or bias list are left out of the
 * tiles (they are ranked in Stage 2).  `rows_per_req` maps row r to
 * request r / rows_per_req (1 for sampling).  req and aux may be NULL; with
 * req the launch also ranks the rows' listed tokens into the workspace,
 * which makes it the same launch as the sampling step's first one. */
int ss_tile_topk(const void* logits, int dtype, int rows, int V, int64_t ld, int rows_per_req,
                 const ss_req* req, const ss_aux* aux, int32_t* out_ids,
                 void* ws, size_t ws_bytes, void* stream);

/* LM head fused with sampling (SonicSampler section 2, "Fused sampling
 * kernels": FlashSampling performs the vocabulary projection and the
 * sampling in one pass, so the logits never reach memory).
 *   hidden [B, ldh] bf16 (raw 16-bit patterns), D used per row;
 *   weight [V, ldw] bf16, one row of D values per vocabulary token;
 *   logits z[b, v] = sum_d hidden[b, d] * weight[v, d], the products exact
 *   and summed in fp32 on the matrix cores (v_mfma_f32_32x32x16_bf16, k in
 *   ascending steps of 16; the summation order inside a step is the
 *   hardware's).  Every entry point below computes a given z[b, v] with the
 *   same instruction sequence, so they all see the same fp32 values.
 * Requirements (else SS_ERR_UNSUPPORTED): D a multiple of 128, D <= 65536,
 * ldh and ldw multiples of 8, hidden and weight 16-byte aligned.
 * ldh < D or ldw < D, a NULL pointer with B > 0: SS_ERR_INVALID_ARG. */

/* Bytes of workspace ss_lmhead_sample_step needs (256-byte aligned, no
 * initialisation): B * V * 4 (logits of the probe columns, and of the
 * other columns for rows whose candidates overflow) + B * 4096 * 8
 * (candidate lists) + the tile stage's share; 0 for B < 0 or V outside
 * [1, SS_V_MAX]. */
size_t ss_lmhead_workspace_bytes(int B, int V);

/* The logits alone: out_logits [B, ldo] fp32 (ldo >= V), z[b, v] at
 * out_logits[b * ldo + v].  Together with ss_sample_step (dtype SS_F32, aux
 * NULL) it is the unfused form of ss_lmhead_sample_step. */
int ss_lmhead_logits(const void* hidden, int64_t ldh, const void* weight, int64_t ldw, int B, int D, int V,
                     float* out_logits, int64_t ldo, void* stream);

/* Sampling straight from the hidden states: the same outputs, statuses,
 * generator use (rng, rng_advance) and noise as ss_sample_step applied to
 * the fp32 logits z with aux = NULL; req[b] as there.  Requests that ask for
 * a grammar mask or name prior or bias entries are SS_ROW_INVALID (no side
 * lists here).  The first P columns (P = V when V <= 16384, else whole
 * tiles of 16384 covering at least 16384 and V / 16) are computed first
 * and give each row its 128 best there; the 128th of them bounds from
 * below the row's 128th best overall, so the GEMM over the other columns
 * keeps only the tokens above it (up to 4096 per row, about (V / P - 1) *
 * 128 on typical rows) and writes no logits.  A row with more (e.g. tied,
 * or peaked far from the first columns) has its other logits stored in the
 * workspace and selected from there.  ws: at least
 * ss_lmhead_workspace_bytes(B, V) bytes.  Errors as ss_sample_step plus the
 * LM-head requirements above. */
int ss_lmhead_sample_step(const void* hidden, int64_t ldh, const void* weight, int64_t ldw, int B, int D, int V,
                          const ss_req* req, ss_rng* rng, uint64_t rng_advance, int32_t* out_tokens,
                          int32_t* out_topk_ids, float* out_probs, int32_t* out_kept, float* out_mass,
                          int32_t* out_status, void* ws, size_t ws_bytes, void* stream);

/* The bandwidth reference of the measurements: reads every byte of the
 * device buffer [p, p + bytes) once with 16-byte loads (p 16-byte aligned,
 * bytes a multiple of 16) on `nblocks` workgroups of 256 threads, and
 * writes out[b] (device, [nblocks] uint32) = the xor of every 32-bit word of
 * the 16-byte words i with (i mod 256*nblocks) / 256 == b.  No other
 * effect. */
int ss_stream_read(const void* p, size_t bytes, int nblocks, uint32_t* out, void* stream);

/* The sampling epilogue's written functions, for checking them against an
 * independent implementation over their whole domains (diagnostic; the
 * same inline device functions the sampling kernels call).  Element i
 * (0 <= i < n <= 2^32) takes the 32-bit argument a = first + i (mod 2^32)
 * and out[i] (device, [n] uint32) receives the result's bit pattern:
 *   SS_SPEC_EXP          exp of the float with bits a, for the arguments
 *                        x = v_k - v_1 <= 0 of the epilogue (ss_sample_step;
 *                        below -86 gives 0; NaN is outside the domain)
 *   SS_SPEC_LOG          ln of the float with bits a (every input)
 *   SS_SPEC_LOG_NORMAL   ln for positive normal finite floats (the
 *                        branch-free form used inside the noise)
 *   SS_SPEC_GUMBEL_WORD  -ln(-ln u) for u = (a + 1/2) 2^-23, the uniform of
 *                        every Philox word whose top 23 bits are a (a < 2^23)
 *   SS_SPEC_PHILOX       the Philox word for counter {a, c1, c2, offset_lo}
 *                        under key {seed_lo, seed_hi ^ offset_hi}
 *   SS_SPEC_GUMBEL       the Gumbel noise for that counter
 * Errors: SS_ERR_INVALID_ARG for an unknown fn, n outside [0, 2^32] or a
 * NULL out with n > 0. */
enum {
    SS_SPEC_EXP = 0,
    SS_SPEC_LOG = 1,
    SS_SPEC_LOG_NORMAL = 2,
    SS_SPEC_GUMBEL_WORD = 3,
    SS_SPEC_PHILOX = 4,
    SS_SPEC_GUMBEL = 5
};
int ss_spec_eval(int fn, uint32_t first, int64_t n, uint32_t c1, uint32_t c2, uint64_t seed, uint64_t offset,
                 uint32_t* out, void* stream);

/* rng->offset += delta on the device (one tiny kernel; capturable). */
int ss_rng_advance(ss_rng* rng, uint64_t delta, void* stream);

/* Static description of a status code. */
const char* ss_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* SS_H */
