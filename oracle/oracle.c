/*
 * CPU oracle for the fused LLM sampling and speculative-verification path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * statement of what the sampler computes.  Only the test-suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it.  It shares no
 * code, header, table or constant generator with the HIP library; both sides
 * are written independently from the same written contract.
 *
 * Sources (web pages on the method):
 *  [SS]  "SonicSampler: Unified Tile-Aware Kernels for LLM Sampling and
 *        Speculative Verification" (arXiv 2607.20475), section 3.1
 *        "Background": logits processing, probability truncation, top-k
 *        selection primitives, sampling (Gumbel-max), speculative
 *        verification; section 3.3 (bounded k = 128).
 *  [DN]  "Decoding and sampling" notes (dl-note, decoding page): sections
 *        "Temperature", "Top-k Sampling", "Top-p (Nucleus) Sampling",
 *        "Min-p", "Combination order", "Rejection Sampler".
 *  [P11] Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
 *        1, 2, 3", SC'11 (Philox4x32-10).
 *  [CW]  Cody & Waite, "Software Manual for the Elementary Functions" (1980):
 *        additive range reduction with a split ln 2.
 *
 * Floating point: IEEE-754 binary32, round to nearest even, no contraction
 * (build with -ffp-contract=off), denormals kept.  Every fused multiply-add
 * below is an explicit fmaf().
 *
 * Parity pins live in tests/ (see the test docstrings): Philox against the
 * Random123 known-answer vectors and rocRAND's host implementation,
 * exp/log against float64 libm, ordering against library sorts, truncation
 * sets against float64 recomputation, sampling and verification against
 * chi-square and closed-form acceptance rates.
 */
#define _GNU_SOURCE
#include <float.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- per-request flag bits (the library's documented bit layout) ---- */
#define OF_GREEDY   (1u << 0)
#define OF_GRAMMAR  (1u << 1)
#define OF_REP      (1u << 2)
#define OF_FREQPRES (1u << 3)
#define OF_BIAS     (1u << 4)
#define OF_TOPK     (1u << 5)
#define OF_TOPP     (1u << 6)
#define OF_MINP     (1u << 7)
#define OF_DRAFT_HIST (1u << 8)
#define SS_ORACLE_GMAX 16   /* largest number of drafts per request */

#define OK_MAX 128           /* bounded candidate set, [SS] section 3.3 */

#define OST_OK 0
#define OST_ALL_MASKED 1
#define OST_INVALID 2
#define OST_TOPK_CLAMPED 3

/* The oracle's own request record (plain fields, no packing). */
typedef struct {
    uint32_t flags;
    float temperature;
    int32_t top_k;
    float top_p;
    float min_p;
    float rep;
    float freq;
    float pres;
    int32_t n_prior;
    int32_t n_bias;
} oreq;

static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* ======================================================================
 * Philox4x32-10 [P11]: ten rounds of the 4x32 Philox S-box.  Each round
 * multiplies counter words 0 and 2 by the two round multipliers, swaps the
 * halves of the 64-bit products across the lanes and XORs in the key; the
 * key is bumped by the two Weyl constants between rounds.
 * ====================================================================== */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t prod0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
        uint64_t prod1 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
        uint32_t n0 = (uint32_t)(prod1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)prod1;
        uint32_t n2 = (uint32_t)(prod0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)prod0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* ======================================================================
 * Spec elementary functions, written from [CW] and the Taylor series.
 * ====================================================================== */

/* exp(x) for x <= 0 (the sampler only needs that range).
 * x = n ln2 + r with n = rint(x log2 e), r reduced with a two-part ln 2;
 * e^r by its degree-7 Taylor polynomial (Horner, fmaf); result p * 2^n.
 * Arguments below -86 return 0, so no result is subnormal. */
float oracle_exp_spec(float x)
{
    if (isnan(x)) return x;
    if (x < -86.0f) return 0.0f;           /* includes -inf */
    if (x > 88.0f) return INFINITY;
    const float log2e = 0x1.715476p+0f;
    const float ln2_hi = 0x1.62e4p-1f;     /* 16 significant bits: n*ln2_hi exact */
    const float ln2_lo = 0x1.7f7d1cp-20f;  /* ln 2 - ln2_hi */
    float n = rintf(x * log2e);
    float r = fmaf(-n, ln2_hi, x);
    r = fmaf(-n, ln2_lo, r);
    float p = 0x1.a01a02p-13f;             /* 1/7! */
    p = fmaf(p, r, 0x1.6c16c2p-10f);       /* 1/6! */
    p = fmaf(p, r, 0x1.111112p-7f);        /* 1/5! */
    p = fmaf(p, r, 0x1.555556p-5f);        /* 1/4! */
    p = fmaf(p, r, 0x1.555556p-3f);        /* 1/3! */
    p = fmaf(p, r, 0.5f);                  /* 1/2! */
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)n);
}

/* ln(x) for x >= 0.  x = 2^e m with m in (sqrt(1/2), sqrt(2)];
 * ln m = 2 atanh(s), s = (m-1)/(m+1), by the odd series up to s^9;
 * result e*ln2_hi + (e*ln2_lo + ln m).  Subnormal x is scaled by 2^24 first. */
float oracle_log_spec(float x)
{
    if (isnan(x) || x < 0.0f) return NAN;
    if (x == 0.0f) return -INFINITY;
    if (isinf(x)) return INFINITY;
    int e = 0;
    if (x < 0x1p-126f) { x = x * 0x1p24f; e = -24; }
    uint32_t b = f2u(x);
    e += (int)((b >> 23) & 0xFFu) - 127;
    float m = u2f((b & 0x007FFFFFu) | 0x3F800000u);   /* [1, 2) */
    if (m > 0x1.6a09e6p+0f) { m = m * 0.5f; e += 1; }
    float s = (m - 1.0f) / (m + 1.0f);
    float s2 = s * s;
    float q = 0x1.c71c72p-4f;              /* 1/9 */
    q = fmaf(q, s2, 0x1.24924ap-3f);       /* 1/7 */
    q = fmaf(q, s2, 0x1.99999ap-3f);       /* 1/5 */
    q = fmaf(q, s2, 0x1.555556p-2f);       /* 1/3 */
    float s3 = s * s2;
    float half_ln = fmaf(s3, q, s);
    float lnm = half_ln + half_ln;
    float ef = (float)e;
    float r = fmaf(ef, 0x1.7f7d1cp-20f, lnm);
    r = fmaf(ef, 0x1.62e4p-1f, r);
    return r;
}

/* Uniform in (0,1) from a 32-bit Philox word: the top 23 bits, centred. */
float oracle_uniform(uint32_t w)
{
    return ((float)(w >> 9) + 0.5f) * 0x1p-23f;
}

/* One Philox word for counter (c0, c1, c2, offset_lo) and key
 * (seed_lo, seed_hi ^ offset_hi). */
uint32_t oracle_philox_word(uint64_t seed, uint64_t offset, uint32_t c0, uint32_t c1, uint32_t c2)
{
    uint32_t ctr[4] = {c0, c1, c2, (uint32_t)offset};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32) ^ (uint32_t)(offset >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    return out[0];
}

/* Standard Gumbel noise -ln(-ln u) for the token with counter (c0,c1,c2). */
float oracle_gumbel(uint64_t seed, uint64_t offset, uint32_t c0, uint32_t c1, uint32_t c2)
{
    float u = oracle_uniform(oracle_philox_word(seed, offset, c0, c1, c2));
    return -oracle_log_spec(-oracle_log_spec(u));
}

/* ======================================================================
 * Logits processing [SS 3.1 "Logits processing"]: grammar mask, repetition
 * penalty, frequency and presence penalties, logit bias, applied in that
 * order to the raw values; the result is then made canonical.
 * ====================================================================== */

static float widen(const void* row, int dtype, int i)
{
    if (dtype == 1) {
        uint16_t h = ((const uint16_t*)row)[i];
        return u2f((uint32_t)h << 16);
    }
    return ((const float*)row)[i];
}

/* NaN -> -inf, +inf -> largest finite float, -0 -> +0. */
static float canon(float z)
{
    if (isnan(z)) return -INFINITY;
    if (z == INFINITY) return FLT_MAX;
    if (z == 0.0f) return 0.0f;
    return z;
}

void oracle_prelude_row(const void* row, int dtype, int V, uint32_t flags,
                        const uint32_t* bitmask_row,
                        const int32_t* prior_ids, const int32_t* prior_cnt, int n_prior,
                        const int32_t* bias_ids, const float* bias_val, int n_bias,
                        float rep, float freq, float pres, float* z)
{
    for (int i = 0; i < V; ++i) {
        z[i] = widen(row, dtype, i);
        if ((flags & OF_GRAMMAR) && !((bitmask_row[i >> 5] >> (i & 31)) & 1u))
            z[i] = -INFINITY;
    }
    /* repetition penalty (CTRL style): shrink positive logits, push negative ones down */
    if (flags & OF_REP) {
        for (int j = 0; j < n_prior; ++j) {
            int id = prior_ids[j];
            if (prior_cnt[j] < 1 || id < 0 || id >= V) continue;
            z[id] = (z[id] > 0.0f) ? z[id] / rep : z[id] * rep;
        }
    }
    /* frequency (per occurrence) and presence (once) penalties */
    if (flags & OF_FREQPRES) {
        for (int j = 0; j < n_prior; ++j) {
            int id = prior_ids[j];
            if (prior_cnt[j] < 1 || id < 0 || id >= V) continue;
            float pen = (float)prior_cnt[j] * freq + pres;
            z[id] = z[id] - pen;
        }
    }
    if (flags & OF_BIAS) {
        for (int j = 0; j < n_bias; ++j) {
            int id = bias_ids[j];
            if (id < 0 || id >= V) continue;
            z[id] = z[id] + bias_val[j];
        }
    }
    for (int i = 0; i < V; ++i) z[i] = canon(z[i]);
}

/* ======================================================================
 * Ordering: i before j iff z_i > z_j, or z_i == z_j and i < j.
 * ====================================================================== */
typedef struct { float z; int32_t id; } zid;

static int zid_cmp(const void* a, const void* b)
{
    const zid* x = (const zid*)a;
    const zid* y = (const zid*)b;
    if (x->z > y->z) return -1;
    if (x->z < y->z) return 1;
    return (x->id < y->id) ? -1 : (x->id > y->id);
}

/* Sorts all V tokens of a row and keeps the first `keep`. */
static void rank_row(const float* z, int V, int keep, zid* work, zid* out)
{
    for (int i = 0; i < V; ++i) { work[i].z = z[i]; work[i].id = i; }
    qsort(work, (size_t)V, sizeof(zid), zid_cmp);
    for (int k = 0; k < keep; ++k) out[k] = work[k];
}

/* ======================================================================
 * Per-row decision: validation, candidate bound, temperature, softmax,
 * top-p / min-p truncation [DN "Temperature", "Top-k", "Top-p", "Min-p",
 * "Combination order"; SS 3.1 "Probability truncation"].
 * ====================================================================== */
typedef struct {
    int status;              /* OST_* */
    int greedy;
    int K;                   /* candidates kept by the bound / top-k */
    int n;                   /* kept after top-p / min-p (stochastic rows) */
    zid cand[OK_MAX];        /* first K tokens in order */
    float v[OK_MAX];         /* z * (1/T), clamped to the finite range */
    float e[OK_MAX];         /* exp(v - v_1) */
    float E[OK_MAX + 1];     /* prefix sums, E[0] = 0 */
} rowdec;

static int finite_f(float x) { return isfinite(x); }

/* Longest lists a request may name (the interface's validity rule: a
 * longer list makes the row invalid, like one longer than its stride). */
#define OPRIOR_MAX 4096
#define OBIAS_MAX 1024

static int lists_fit(const oreq* r, int prior_stride, int bias_stride)
{
    return r->n_prior >= 0 && r->n_prior <= prior_stride && r->n_prior <= OPRIOR_MAX &&
           r->n_bias >= 0 && r->n_bias <= bias_stride && r->n_bias <= OBIAS_MAX;
}

static int validate(const oreq* r, int prior_stride, int bias_stride, const float* bias_val,
                    int* greedy)
{
    uint32_t f = r->flags;
    if (!lists_fit(r, prior_stride, bias_stride)) return 0;
    if ((f & OF_REP) && !(finite_f(r->rep) && r->rep > 0.0f)) return 0;
    if ((f & OF_FREQPRES) && !(finite_f(r->freq) && finite_f(r->pres))) return 0;
    if (f & OF_BIAS)
        for (int j = 0; j < r->n_bias; ++j)
            if (!finite_f(bias_val[j])) return 0;
    int g = (f & OF_GREEDY) != 0;
    if (!g) {
        if (isnan(r->temperature)) return 0;
        if (r->temperature <= 0.0f) g = 1;
        else if ((f & OF_TOPK) && r->top_k == 1) g = 1;
    }
    if (!g) {
        if (!finite_f(r->temperature)) return 0;
        if ((f & OF_TOPK) && r->top_k < 1) return 0;
        if ((f & OF_TOPP) && !(r->top_p > 0.0f && r->top_p <= 1.0f)) return 0;
        if ((f & OF_MINP) && !(r->min_p >= 0.0f && r->min_p <= 1.0f)) return 0;
    }
    *greedy = g;
    return 1;
}

/* z: processed logits of the row.  Fills d. */
static void decide_row(const oreq* r, const float* z, int V, int prior_stride, int bias_stride,
                       const float* bias_val, zid* work, rowdec* d)
{
    memset(d, 0, sizeof(*d));
    int greedy = 0;
    if (!validate(r, prior_stride, bias_stride, bias_val, &greedy)) {
        d->status = OST_INVALID;
        return;
    }
    d->greedy = greedy;
    int K = OK_MAX;
    int clamped = 0;
    if ((r->flags & OF_TOPK) && r->top_k >= 1) {
        if (r->top_k > OK_MAX) clamped = 1;
        else K = r->top_k;
    }
    if (K > V) K = V;
    d->K = K;
    rank_row(z, V, K, work, d->cand);
    d->status = clamped ? OST_TOPK_CLAMPED : OST_OK;
    if (d->cand[0].z == -INFINITY) { d->status = OST_ALL_MASKED; return; }
    if (greedy) { d->n = 1; return; }

    float invT = 1.0f / r->temperature;
    for (int k = 0; k < K; ++k) {
        float zk = d->cand[k].z;
        float v;
        if (zk == -INFINITY) v = -INFINITY;
        else {
            v = zk * invT;
            if (v > FLT_MAX) v = FLT_MAX;
            if (v < -FLT_MAX) v = -FLT_MAX;
        }
        d->v[k] = v;
    }
    float m = d->v[0];
    d->E[0] = 0.0f;
    for (int k = 0; k < K; ++k) {
        d->e[k] = oracle_exp_spec(d->v[k] - m);
        d->E[k + 1] = d->E[k] + d->e[k];     /* left to right */
    }
    float Z = d->E[K];
    int n_p = K;
    if ((r->flags & OF_TOPP) && r->top_p < 1.0f) {
        /* smallest prefix whose mass reaches top_p: keep rank k while the
         * mass strictly before it is below top_p * Z */
        float thr = r->top_p * Z;
        n_p = 0;
        for (int k = 0; k < K; ++k)
            if (d->E[k] < thr) n_p = k + 1;
    }
    int n_m = K;
    if ((r->flags & OF_MINP) && r->min_p > 0.0f) {
        /* p_k >= min_p * p_max  <=>  v_k - v_1 >= ln(min_p)  (no softmax) */
        float L = oracle_log_spec(r->min_p);
        n_m = 0;
        for (int k = 0; k < K; ++k)
            if (d->v[k] - m >= L) ++n_m;
    }
    d->n = n_p < n_m ? n_p : n_m;
}

/* Gumbel-max over the first n candidates [SS 3.1 "Sampling"]:
 * argmax_k v_k + g(id_k); ties go to the lower token id. */
static int32_t gumbel_pick(const rowdec* d, int n, uint64_t seed, uint64_t offset,
                           uint32_t c1, uint32_t c2)
{
    int32_t best = -1;
    float best_s = 0.0f;
    for (int k = 0; k < n; ++k) {
        int32_t id = d->cand[k].id;
        float s = d->v[k] + oracle_gumbel(seed, offset, (uint32_t)id, c1, c2);
        if (best < 0 || s > best_s || (s == best_s && id < best)) { best = id; best_s = s; }
    }
    return best;
}

/* ======================================================================
 * Batched single-step sampling.
 * ====================================================================== */
typedef struct {
    const void* logits; int dtype; int B; int V; int64_t ld;
    const oreq* req;
    const int32_t* prior_ids; const int32_t* prior_cnt; int prior_stride;
    const int32_t* bias_ids; const float* bias_val; int bias_stride;
    const uint32_t* bitmask; int64_t bitmask_stride;
    uint64_t seed, offset;
    int32_t* tokens; int32_t* topk_ids; float* probs; int32_t* kept; float* mass; int32_t* status;
    int row_begin, row_end;
} sample_job;

static const void* row_ptr(const void* base, int dtype, int64_t ld, int64_t r)
{
    return dtype == 1 ? (const void*)((const uint16_t*)base + r * ld)
                      : (const void*)((const float*)base + r * ld);
}

static void prelude_for(const sample_job* J, const oreq* r, int64_t row, int64_t lrow, float* z)
{
    oracle_prelude_row(row_ptr(J->logits, J->dtype, J->ld, row), J->dtype, J->V, r->flags,
                       J->bitmask ? J->bitmask + row * J->bitmask_stride : NULL,
                       J->prior_ids ? J->prior_ids + lrow * J->prior_stride : NULL,
                       J->prior_cnt ? J->prior_cnt + lrow * J->prior_stride : NULL,
                       (r->flags & (OF_REP | OF_FREQPRES)) ? r->n_prior : 0,
                       J->bias_ids ? J->bias_ids + lrow * J->bias_stride : NULL,
                       J->bias_val ? J->bias_val + lrow * J->bias_stride : NULL,
                       (r->flags & OF_BIAS) ? r->n_bias : 0,
                       r->rep, r->freq, r->pres, z);
}

/* A row whose flags need a side array that was not given is invalid. */
static int arrays_ok(const oreq* r, const sample_job* J)
{
    if ((r->flags & OF_GRAMMAR) && !J->bitmask) return 0;
    if ((r->flags & (OF_REP | OF_FREQPRES)) && r->n_prior > 0 && (!J->prior_ids || !J->prior_cnt)) return 0;
    if ((r->flags & OF_BIAS) && r->n_bias > 0 && (!J->bias_ids || !J->bias_val)) return 0;
    return 1;
}

static void* sample_worker(void* arg)
{
    const sample_job* J = (const sample_job*)arg;
    float* z = (float*)malloc(sizeof(float) * (size_t)J->V);
    zid* work = (zid*)malloc(sizeof(zid) * (size_t)J->V);
    rowdec* d = (rowdec*)malloc(sizeof(rowdec));
    for (int b = J->row_begin; b < J->row_end; ++b) {
        const oreq* r = &J->req[b];
        const float* bv = J->bias_val ? J->bias_val + (int64_t)b * J->bias_stride : NULL;
        int valid_shape = lists_fit(r, J->prior_stride, J->bias_stride) && arrays_ok(r, J);
        if (valid_shape) prelude_for(J, r, b, b, z);
        if (valid_shape) decide_row(r, z, J->V, J->prior_stride, J->bias_stride, bv, work, d);
        else { memset(d, 0, sizeof(*d)); d->status = OST_INVALID; }
        int32_t tok = -1;
        float mass = 0.0f;
        int kept = 0;
        if (d->status == OST_OK || d->status == OST_TOPK_CLAMPED) {
            if (d->greedy) { tok = d->cand[0].id; mass = 1.0f; kept = 1; }
            else {
                tok = gumbel_pick(d, d->n, J->seed, J->offset, (uint32_t)b, 0u);
                kept = d->n;
                mass = d->E[d->n] / d->E[d->K];
            }
        }
        J->tokens[b] = tok;
        if (J->status) J->status[b] = d->status;
        if (J->kept) J->kept[b] = kept;
        if (J->mass) J->mass[b] = mass;
        if (J->topk_ids) {
            for (int k = 0; k < OK_MAX; ++k)
                J->topk_ids[(int64_t)b * OK_MAX + k] =
                    (d->status != OST_INVALID && k < d->K) ? d->cand[k].id : -1;
        }
        if (J->probs) {
            for (int k = 0; k < OK_MAX; ++k) {
                float p = 0.0f;
                if (d->status == OST_OK || d->status == OST_TOPK_CLAMPED) {
                    if (d->greedy) p = (k == 0) ? 1.0f : 0.0f;
                    else if (k < d->K) p = d->e[k] / d->E[d->K];
                }
                J->probs[(int64_t)b * OK_MAX + k] = p;
            }
        }
    }
    free(z); free(work); free(d);
    return NULL;
}

static void run_rows(void* (*fn)(void*), void* jobs, size_t job_size, int rows, int threads,
                     void (*set_range)(void*, int, int))
{
    if (threads < 1) threads = 1;
    if (threads > rows) threads = rows > 0 ? rows : 1;
    pthread_t* tid = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)threads);
    for (int t = 0; t < threads; ++t) {
        void* job = (char*)jobs + (size_t)t * job_size;
        int lo = (int)((int64_t)rows * t / threads);
        int hi = (int)((int64_t)rows * (t + 1) / threads);
        set_range(job, lo, hi);
        if (threads == 1) fn(job);
        else pthread_create(&tid[t], NULL, fn, job);
    }
    if (threads > 1)
        for (int t = 0; t < threads; ++t) pthread_join(tid[t], NULL);
    free(tid);
}

static void sample_set_range(void* j, int lo, int hi)
{
    ((sample_job*)j)->row_begin = lo;
    ((sample_job*)j)->row_end = hi;
}

int oracle_sample(const void* logits, int dtype, int B, int V, int64_t ld, const oreq* req,
                  const int32_t* prior_ids, const int32_t* prior_cnt, int prior_stride,
                  const int32_t* bias_ids, const float* bias_val, int bias_stride,
                  const uint32_t* bitmask, int64_t bitmask_stride,
                  uint64_t seed, uint64_t offset,
                  int32_t* tokens, int32_t* topk_ids, float* probs, int32_t* kept, float* mass,
                  int32_t* status, int threads)
{
    if (!logits || !req || !tokens || B < 0 || V < 1 || ld < V) return -1;
    if (threads < 1) threads = 1;
    sample_job* jobs = (sample_job*)calloc((size_t)threads, sizeof(sample_job));
    for (int t = 0; t < threads; ++t) {
        sample_job* J = &jobs[t];
        J->logits = logits; J->dtype = dtype; J->B = B; J->V = V; J->ld = ld; J->req = req;
        J->prior_ids = prior_ids; J->prior_cnt = prior_cnt; J->prior_stride = prior_stride;
        J->bias_ids = bias_ids; J->bias_val = bias_val; J->bias_stride = bias_stride;
        J->bitmask = bitmask; J->bitmask_stride = bitmask_stride;
        J->seed = seed; J->offset = offset;
        J->tokens = tokens; J->topk_ids = topk_ids; J->probs = probs; J->kept = kept;
        J->mass = mass; J->status = status;
    }
    if (B > 0) run_rows(sample_worker, jobs, sizeof(sample_job), B, threads, sample_set_range);
    free(jobs);
    return 0;
}

/* ======================================================================
 * Speculative verification [SS 3.1 "Speculative verification";
 * DN "Rejection Sampler"].  Request b owns target rows b*(gamma+1)+j.
 * Draft token d_j is accepted when q_j(d_j) > 0 and u_j * q_j(d_j) <=
 * p_j(d_j); at the first rejection one token is drawn from the residual
 * max(0, p_j - q_j) and the request stops; when all gamma drafts are
 * accepted a bonus token is drawn from position gamma.
 * Noise counters (c0, c1, c2): Gumbel for position j (0 / token id, b,
 * j), acceptance uniform (0, b, (1<<24)|j), residual Gumbel (id, b,
 * (2<<24)|j).
 * Variable drafts per request [DN "Rejection Sampler": per-request draft
 * counts from cumulative offsets]: with cu_num_draft (inclusive cumulative
 * counts, n_b = cu[b] - cu[b-1]) request b has n_b <= gamma drafts at
 * positions 0..n_b-1 of its (still gamma+1) rows, and its bonus position
 * is n_b; the rows past n_b take no part.  n_b outside [0, gamma] makes
 * the request invalid.
 * Penalty history with the earlier drafts [DN "Repetition penalty",
 * "Frequency and presence penalties": the penalised history is every token
 * generated so far]: for a request with OF_DRAFT_HIST, position j's
 * history is the request's prior list with d_0..d_{j-1} added, each draft
 * (an id in [0, V)) adding one occurrence: to the count of the first prior
 * entry with its id and a count >= 1, else to an entry appended for it
 * (one per distinct id, in order of first appearance).
 * ====================================================================== */
typedef struct {
    const void* target; int dtype; int B; int gamma; int V; int64_t ld;
    const oreq* req;
    const int32_t* prior_ids; const int32_t* prior_cnt; int prior_stride;
    const int32_t* bias_ids; const float* bias_val; int bias_stride;
    const uint32_t* bitmask; int64_t bitmask_stride;
    const int32_t* draft_ids; const float* draft_probs;
    const int32_t* cu_num_draft;
    uint64_t seed, offset;
    int32_t* out_tokens; int32_t* n_emit; int32_t* status;
    int row_begin, row_end;
} verify_job;

static void verify_set_range(void* j, int lo, int hi)
{
    ((verify_job*)j)->row_begin = lo;
    ((verify_job*)j)->row_end = hi;
}

static void* verify_worker(void* arg)
{
    const verify_job* J = (const verify_job*)arg;
    const int G = J->gamma;
    const int V = J->V;
    float* z = (float*)malloc(sizeof(float) * (size_t)V);
    zid* work = (zid*)malloc(sizeof(zid) * (size_t)V);
    rowdec* d = (rowdec*)malloc(sizeof(rowdec));
    int32_t* hist_ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)(J->prior_stride + G + 1));
    int32_t* hist_cnt = (int32_t*)malloc(sizeof(int32_t) * (size_t)(J->prior_stride + G + 1));
    sample_job S;            /* reuse the prelude helper */
    memset(&S, 0, sizeof(S));
    S.logits = J->target; S.dtype = J->dtype; S.V = V; S.ld = J->ld;
    S.prior_ids = J->prior_ids; S.prior_cnt = J->prior_cnt; S.prior_stride = J->prior_stride;
    S.bias_ids = J->bias_ids; S.bias_val = J->bias_val; S.bias_stride = J->bias_stride;
    S.bitmask = J->bitmask; S.bitmask_stride = J->bitmask_stride;

    for (int b = J->row_begin; b < J->row_end; ++b) {
        const oreq* r = &J->req[b];
        int32_t* out = J->out_tokens + (int64_t)b * (G + 1);
        for (int j = 0; j <= G; ++j) out[j] = -1;
        int emitted = 0;
        int st = OST_OK;
        const float* bv = J->bias_val ? J->bias_val + (int64_t)b * J->bias_stride : NULL;
        if (!lists_fit(r, J->prior_stride, J->bias_stride) || !arrays_ok(r, &S)) {
            st = OST_INVALID;
        }
        /* this request's draft count: gamma, or from the cumulative offsets */
        int Gb = G;
        if (J->cu_num_draft) {
            const int64_t hi = J->cu_num_draft[b];
            const int64_t lo = b > 0 ? J->cu_num_draft[b - 1] : 0;
            if (hi - lo < 0 || hi - lo > G) st = OST_INVALID;
            else Gb = (int)(hi - lo);
        }
        for (int j = 0; j <= Gb && st != OST_INVALID; ++j) {
            int64_t row = (int64_t)b * (G + 1) + j;
            if ((r->flags & OF_DRAFT_HIST) && (r->flags & (OF_REP | OF_FREQPRES)) && j > 0) {
                /* the prior entries, then the drafts before position j */
                const int np = r->n_prior;
                for (int k = 0; k < np; ++k) {
                    hist_ids[k] = J->prior_ids[(int64_t)b * J->prior_stride + k];
                    hist_cnt[k] = J->prior_cnt[(int64_t)b * J->prior_stride + k];
                }
                int nh = np;
                for (int i = 0; i < j; ++i) {
                    const int32_t dv = J->draft_ids[(int64_t)b * G + i];
                    if (dv < 0 || dv >= V) continue;
                    int k = 0;
                    while (k < nh && !(hist_ids[k] == dv && hist_cnt[k] >= 1)) ++k;
                    if (k < nh) { hist_cnt[k] += 1; continue; }
                    hist_ids[nh] = dv;
                    hist_cnt[nh] = 1;
                    ++nh;
                }
                oracle_prelude_row(row_ptr(S.logits, S.dtype, S.ld, row), S.dtype, V, r->flags,
                                   S.bitmask ? S.bitmask + row * S.bitmask_stride : NULL,
                                   hist_ids, hist_cnt, nh,
                                   S.bias_ids ? S.bias_ids + (int64_t)b * S.bias_stride : NULL,
                                   S.bias_val ? S.bias_val + (int64_t)b * S.bias_stride : NULL,
                                   (r->flags & OF_BIAS) ? r->n_bias : 0,
                                   r->rep, r->freq, r->pres, z);
            } else {
                prelude_for(&S, r, row, b, z);
            }
            decide_row(r, z, V, J->prior_stride, J->bias_stride, bv, work, d);
            if (d->status == OST_INVALID) { st = OST_INVALID; emitted = 0; break; }
            if (d->status == OST_TOPK_CLAMPED) st = OST_TOPK_CLAMPED;
            if (d->status == OST_ALL_MASKED) { st = OST_ALL_MASKED; break; }
            if (j == Gb) {   /* bonus token */
                out[emitted++] = d->greedy ? d->cand[0].id
                                           : gumbel_pick(d, d->n, J->seed, J->offset, (uint32_t)b, (uint32_t)Gb);
                break;
            }
            int32_t dj = J->draft_ids[(int64_t)b * G + j];
            if (d->greedy) {
                int32_t a = d->cand[0].id;
                if (dj == a) { out[emitted++] = dj; continue; }
                out[emitted++] = a;
                break;
            }
            const float* q = J->draft_probs + ((int64_t)b * G + j) * V;
            float En = d->E[d->n];
            float p_d = 0.0f;
            for (int k = 0; k < d->n; ++k)
                if (d->cand[k].id == dj) p_d = d->e[k] / En;
            float q_d = (dj >= 0 && dj < V) ? q[dj] : 0.0f;
            float u = oracle_uniform(oracle_philox_word(J->seed, J->offset, 0u, (uint32_t)b,
                                                        (1u << 24) | (uint32_t)j));
            if (q_d > 0.0f && u * q_d <= p_d) { out[emitted++] = dj; continue; }
            /* rejected: residual max(0, p - q) over the kept candidates */
            int32_t best = -1;
            float best_s = 0.0f;
            for (int k = 0; k < d->n; ++k) {
                int32_t id = d->cand[k].id;
                float rho = d->e[k] / En - q[id];
                if (!(rho > 0.0f)) continue;
                float s = oracle_log_spec(rho) +
                          oracle_gumbel(J->seed, J->offset, (uint32_t)id, (uint32_t)b, (2u << 24) | (uint32_t)j);
                if (best < 0 || s > best_s || (s == best_s && id < best)) { best = id; best_s = s; }
            }
            if (best < 0)   /* p <= q everywhere on the kept set: draw from p */
                best = gumbel_pick(d, d->n, J->seed, J->offset, (uint32_t)b, (2u << 24) | (uint32_t)j);
            out[emitted++] = best;
            break;
        }
        if (st == OST_INVALID) { for (int j = 0; j <= G; ++j) out[j] = -1; emitted = 0; }
        J->n_emit[b] = emitted;
        if (J->status) J->status[b] = st;
    }
    free(z); free(work); free(d); free(hist_ids); free(hist_cnt);
    return NULL;
}

int oracle_verify(const void* target, int dtype, int B, int gamma, int V, int64_t ld, const oreq* req,
                  const int32_t* prior_ids, const int32_t* prior_cnt, int prior_stride,
                  const int32_t* bias_ids, const float* bias_val, int bias_stride,
                  const uint32_t* bitmask, int64_t bitmask_stride,
                  const int32_t* draft_ids, const float* draft_probs, const int32_t* cu_num_draft,
                  uint64_t seed, uint64_t offset,
                  int32_t* out_tokens, int32_t* n_emit, int32_t* status, int threads)
{
    if (!target || !req || !draft_ids || !draft_probs || !out_tokens || !n_emit) return -1;
    if (B < 0 || gamma < 1 || V < 1 || ld < V) return -1;
    if (threads < 1) threads = 1;
    verify_job* jobs = (verify_job*)calloc((size_t)threads, sizeof(verify_job));
    for (int t = 0; t < threads; ++t) {
        verify_job* J = &jobs[t];
        J->target = target; J->dtype = dtype; J->B = B; J->gamma = gamma; J->V = V; J->ld = ld;
        J->req = req;
        J->prior_ids = prior_ids; J->prior_cnt = prior_cnt; J->prior_stride = prior_stride;
        J->bias_ids = bias_ids; J->bias_val = bias_val; J->bias_stride = bias_stride;
        J->bitmask = bitmask; J->bitmask_stride = bitmask_stride;
        J->draft_ids = draft_ids; J->draft_probs = draft_probs; J->cu_num_draft = cu_num_draft;
        J->seed = seed; J->offset = offset;
        J->out_tokens = out_tokens; J->n_emit = n_emit; J->status = status;
    }
    if (B > 0) run_rows(verify_worker, jobs, sizeof(verify_job), B, threads, verify_set_range);
    free(jobs);
    return 0;
}

/* ======================================================================
 * Dense verification [DN "Rejection Sampler": the notes' rejection and
 * recovery kernels take full-vocabulary target probabilities (and draft
 * probabilities, or none: then the draft probability counts as 1 and the
 * recovered token is drawn from the target distribution with the draft
 * token left out); the recovered token is the argmax of the residual over
 * an exponential race, i.e. a Gumbel-max on its logarithm].
 * p_j is the softmax of v = z/T over the whole vocabulary, z the canonical
 * logits: no truncation (top-k, top-p and min-p settings do not apply) and
 * no other processing, so a request that asks for a grammar mask, penalties
 * or a bias list is invalid here.  Greedy: SS_GREEDY or T <= 0; otherwise
 * T must be finite.  v_i = z_i * (1/T) clamped to the finite range (-inf
 * stays -inf), m = max_i v_i, e_i = exp(v_i - m) with the written exp,
 * Z = sum_i e_i (double, rounded once to float), p_i = e_i / Z.
 *   accept d_j:   q_j(d_j) > 0 and u_j q_j(d_j) <= p_j(d_j)
 *   recovered:    argmax over r_i = p_i - q_j(i) > 0 (no draft
 *                 probabilities: r_i = p_i, with r = 0 at d_j) of
 *                 ln r_i + g(i, b, (2<<24)|j); no such i: argmax of
 *                 v_i + g(i, b, (2<<24)|j)
 *   bonus:        argmax of v_i + g(i, b, n_b) over the whole vocabulary
 *   greedy rows:  accept iff d_j is the best id; emit the best id
 *   a row whose every value is -inf: status ALL_MASKED, stop.
 * Noise counters as in the bounded verification.  `fragile[b]` is set when
 * the emitted tokens change if Z is taken as Z (1 - zslack) or Z (1 + zslack)
 * instead: a sum of V terms in another order may differ from this one by
 * about that much, and only such requests may legitimately differ.
 * ====================================================================== */
typedef struct {
    const void* target; int dtype; int B; int gamma; int V; int64_t ld;
    const oreq* req;
    const int32_t* draft_ids; const float* draft_probs; const int32_t* cu_num_draft;
    uint64_t seed, offset;
    double zslack;
    int32_t* out_tokens; int32_t* n_emit; int32_t* status; int32_t* fragile;
    int row_begin, row_end;
} dense_job;

static void dense_set_range(void* j, int lo, int hi)
{
    ((dense_job*)j)->row_begin = lo;
    ((dense_job*)j)->row_end = hi;
}

/* One request's tokens with Z scaled by zscale; returns the status. */
static int dense_request(const dense_job* J, int b, int greedy, int Gb, double zscale,
                         float* z, float* v, float* e, int32_t* out, int* emitted)
{
    const int G = J->gamma, V = J->V;
    const oreq* r = &J->req[b];
    *emitted = 0;
    for (int j = 0; j <= Gb; ++j) {
        const int64_t row = (int64_t)b * (G + 1) + j;
        const void* rp = row_ptr(J->target, J->dtype, J->ld, row);
        for (int i = 0; i < V; ++i) z[i] = canon(widen(rp, J->dtype, i));
        const int32_t d = j < Gb ? J->draft_ids[(int64_t)b * G + j] : -1;
        if (greedy) {
            int best = 0;
            for (int i = 1; i < V; ++i)
                if (z[i] > z[best]) best = i;
            if (z[best] == -INFINITY) return OST_ALL_MASKED;
            out[(*emitted)++] = (j == Gb || d != best) ? best : d;
            if (j == Gb || d != best) return OST_OK;
            continue;
        }
        const float invT = 1.0f / r->temperature;
        float m = -INFINITY;
        for (int i = 0; i < V; ++i) {
            float vi;
            if (z[i] == -INFINITY) vi = -INFINITY;
            else {
                vi = z[i] * invT;
                if (vi > FLT_MAX) vi = FLT_MAX;
                if (vi < -FLT_MAX) vi = -FLT_MAX;
            }
            v[i] = vi;
            if (vi > m) m = vi;
        }
        if (m == -INFINITY) return OST_ALL_MASKED;
        double Zd = 0.0;
        for (int i = 0; i < V; ++i) {
            e[i] = oracle_exp_spec(v[i] - m);
            Zd += (double)e[i];
        }
        const float Z = (float)(Zd * zscale);
        if (j == Gb) {   /* bonus: the untruncated target distribution */
            int32_t best = -1;
            float bs = 0.0f;
            for (int i = 0; i < V; ++i) {
                float s = v[i] + oracle_gumbel(J->seed, J->offset, (uint32_t)i, (uint32_t)b, (uint32_t)Gb);
                if (best < 0 || s > bs) { best = i; bs = s; }
            }
            out[(*emitted)++] = best;
            return OST_OK;
        }
        const float* q = J->draft_probs ? J->draft_probs + ((int64_t)b * G + j) * V : NULL;
        const int din = d >= 0 && d < V;
        const float q_d = din ? (q ? q[d] : 1.0f) : 0.0f;
        const float p_d = din ? e[d] / Z : 0.0f;
        const float u = oracle_uniform(oracle_philox_word(J->seed, J->offset, 0u, (uint32_t)b,
                                                          (1u << 24) | (uint32_t)j));
        if (q_d > 0.0f && u * q_d <= p_d) { out[(*emitted)++] = d; continue; }
        const uint32_t c2 = (2u << 24) | (uint32_t)j;
        int32_t best = -1;
        float bs = 0.0f;
        for (int i = 0; i < V; ++i) {
            const float pi = e[i] / Z;
            const float rho = q ? pi - q[i] : (i == d ? 0.0f : pi);
            if (!(rho > 0.0f)) continue;
            const float s = oracle_log_spec(rho) + oracle_gumbel(J->seed, J->offset, (uint32_t)i, (uint32_t)b, c2);
            if (best < 0 || s > bs) { best = i; bs = s; }
        }
        if (best < 0) {   /* p <= q everywhere: draw from p */
            for (int i = 0; i < V; ++i) {
                const float s = v[i] + oracle_gumbel(J->seed, J->offset, (uint32_t)i, (uint32_t)b, c2);
                if (best < 0 || s > bs) { best = i; bs = s; }
            }
        }
        out[(*emitted)++] = best;
        return OST_OK;
    }
    return OST_OK;
}

static void* dense_worker(void* arg)
{
    const dense_job* J = (const dense_job*)arg;
    const int G = J->gamma, V = J->V;
    float* z = (float*)malloc(sizeof(float) * (size_t)V);
    float* v = (float*)malloc(sizeof(float) * (size_t)V);
    float* e = (float*)malloc(sizeof(float) * (size_t)V);
    int32_t alt[2][SS_ORACLE_GMAX + 1];
    for (int b = J->row_begin; b < J->row_end; ++b) {
        const oreq* r = &J->req[b];
        int32_t* out = J->out_tokens + (int64_t)b * (G + 1);
        for (int j = 0; j <= G; ++j) out[j] = -1;
        int st = OST_OK, emitted = 0, fragile = 0;
        int greedy = (r->flags & OF_GREEDY) != 0;
        if (r->flags & (OF_GRAMMAR | OF_REP | OF_FREQPRES | OF_BIAS | OF_DRAFT_HIST)) st = OST_INVALID;
        if (!greedy) {
            if (isnan(r->temperature)) st = OST_INVALID;
            else if (r->temperature <= 0.0f) greedy = 1;
            else if (!finite_f(r->temperature)) st = OST_INVALID;
        }
        int Gb = G;
        if (J->cu_num_draft) {
            const int64_t hi = J->cu_num_draft[b];
            const int64_t lo = b > 0 ? J->cu_num_draft[b - 1] : 0;
            if (hi - lo < 0 || hi - lo > G) st = OST_INVALID;
            else Gb = (int)(hi - lo);
        }
        if (st != OST_INVALID) {
            st = dense_request(J, b, greedy, Gb, 1.0, z, v, e, out, &emitted);
            if (!greedy && J->zslack > 0.0) {
                for (int s = 0; s < 2; ++s) {
                    int em2 = 0;
                    for (int j = 0; j <= G; ++j) alt[s][j] = -1;
                    int st2 = dense_request(J, b, 0, Gb, s ? 1.0 + J->zslack : 1.0 - J->zslack, z, v, e, alt[s], &em2);
                    if (st2 != st || em2 != emitted || memcmp(alt[s], out, sizeof(int32_t) * (size_t)(G + 1)) != 0)
                        fragile = 1;
                }
            }
        }
        if (st == OST_INVALID) { for (int j = 0; j <= G; ++j) out[j] = -1; emitted = 0; }
        J->n_emit[b] = emitted;
        if (J->status) J->status[b] = st;
        if (J->fragile) J->fragile[b] = fragile;
    }
    free(z); free(v); free(e);
    return NULL;
}

int oracle_verify_dense(const void* target, int dtype, int B, int gamma, int V, int64_t ld, const oreq* req,
                        const int32_t* draft_ids, const float* draft_probs, const int32_t* cu_num_draft,
                        uint64_t seed, uint64_t offset, double zslack,
                        int32_t* out_tokens, int32_t* n_emit, int32_t* status, int32_t* fragile, int threads)
{
    if (!target || !req || !draft_ids || !out_tokens || !n_emit) return -1;
    if (B < 0 || gamma < 1 || gamma > SS_ORACLE_GMAX || V < 1 || ld < V) return -1;
    if (threads < 1) threads = 1;
    dense_job* jobs = (dense_job*)calloc((size_t)threads, sizeof(dense_job));
    for (int t = 0; t < threads; ++t) {
        dense_job* J = &jobs[t];
        J->target = target; J->dtype = dtype; J->B = B; J->gamma = gamma; J->V = V; J->ld = ld;
        J->req = req; J->draft_ids = draft_ids; J->draft_probs = draft_probs; J->cu_num_draft = cu_num_draft;
        J->seed = seed; J->offset = offset; J->zslack = zslack;
        J->out_tokens = out_tokens; J->n_emit = n_emit; J->status = status; J->fragile = fragile;
    }
    if (B > 0) run_rows(dense_worker, jobs, sizeof(dense_job), B, threads, dense_set_range);
    free(jobs);
    return 0;
}

/* ======================================================================
 * Plain top-k [SS 3.1 "Top-k selection primitives"]: the first k tokens in
 * order of the canonical raw values, with their values.  Positions past V
 * hold id -1 and value -inf.
 * ====================================================================== */
typedef struct {
    const void* logits; int dtype; int V; int64_t ld; int k;
    int32_t* ids; float* vals;
    int row_begin, row_end;
} topk_job;

static void topk_set_range(void* j, int lo, int hi)
{
    ((topk_job*)j)->row_begin = lo;
    ((topk_job*)j)->row_end = hi;
}

static void* topk_worker(void* arg)
{
    const topk_job* J = (const topk_job*)arg;
    float* z = (float*)malloc(sizeof(float) * (size_t)J->V);
    zid* work = (zid*)malloc(sizeof(zid) * (size_t)J->V);
    zid* top = (zid*)malloc(sizeof(zid) * (size_t)(J->k > 0 ? J->k : 1));
    int keep = J->k < J->V ? J->k : J->V;
    for (int b = J->row_begin; b < J->row_end; ++b) {
        const void* row = row_ptr(J->logits, J->dtype, J->ld, b);
        for (int i = 0; i < J->V; ++i) z[i] = canon(widen(row, J->dtype, i));
        rank_row(z, J->V, keep, work, top);
        for (int k = 0; k < J->k; ++k) {
            J->ids[(int64_t)b * J->k + k] = k < keep ? top[k].id : -1;
            if (J->vals) J->vals[(int64_t)b * J->k + k] = k < keep ? top[k].z : -INFINITY;
        }
    }
    free(z); free(work); free(top);
    return NULL;
}

int oracle_topk(const void* logits, int dtype, int B, int V, int64_t ld, int k,
                int32_t* ids, float* vals, int threads)
{
    if (!logits || !ids || B < 0 || V < 1 || ld < V || k < 1 || k > OK_MAX) return -1;
    if (threads < 1) threads = 1;
    topk_job* jobs = (topk_job*)calloc((size_t)threads, sizeof(topk_job));
    for (int t = 0; t < threads; ++t) {
        jobs[t].logits = logits; jobs[t].dtype = dtype; jobs[t].V = V; jobs[t].ld = ld;
        jobs[t].k = k; jobs[t].ids = ids; jobs[t].vals = vals;
    }
    if (B > 0) run_rows(topk_worker, jobs, sizeof(topk_job), B, threads, topk_set_range);
    free(jobs);
    return 0;
}

/* ======================================================================
 * Tile view [SS 3.2, Fig. 1 stage 1]: for vocabulary tiles of `tile`
 * tokens, the first 128 tokens of each tile in order of the processed
 * logits, leaving out every token named by an active penalty or bias list
 * (those are ranked in the merge stage).  Positions without a token hold
 * -1.  `rows_per_req` maps row r to request r / rows_per_req.
 * ====================================================================== */
int oracle_tile_topk(const void* logits, int dtype, int rows, int V, int64_t ld, int tile,
                     int rows_per_req, const oreq* req,
                     const int32_t* prior_ids, const int32_t* prior_cnt, int prior_stride,
                     const int32_t* bias_ids, const float* bias_val, int bias_stride,
                     const uint32_t* bitmask, int64_t bitmask_stride, int32_t* out_ids)
{
    if (!logits || !out_ids || rows < 0 || V < 1 || tile < 1 || rows_per_req < 1) return -1;
    int Zv = (V + tile - 1) / tile;
    float* z = (float*)malloc(sizeof(float) * (size_t)V);
    zid* work = (zid*)malloc(sizeof(zid) * (size_t)tile);
    unsigned char* listed = (unsigned char*)malloc((size_t)V);
    sample_job S;
    memset(&S, 0, sizeof(S));
    S.logits = logits; S.dtype = dtype; S.V = V; S.ld = ld;
    S.prior_ids = prior_ids; S.prior_cnt = prior_cnt; S.prior_stride = prior_stride;
    S.bias_ids = bias_ids; S.bias_val = bias_val; S.bias_stride = bias_stride;
    S.bitmask = bitmask; S.bitmask_stride = bitmask_stride;
    for (int r = 0; r < rows; ++r) {
        int b = r / rows_per_req;
        oreq q = req ? req[b] : (oreq){0};
        if (q.n_prior < 0 || q.n_prior > prior_stride || q.n_prior > OPRIOR_MAX) q.n_prior = 0;
        if (q.n_bias < 0 || q.n_bias > bias_stride || q.n_bias > OBIAS_MAX) q.n_bias = 0;
        prelude_for(&S, &q, r, b, z);
        memset(listed, 0, (size_t)V);
        if (q.flags & (OF_REP | OF_FREQPRES))
            for (int j = 0; j < q.n_prior; ++j) {
                int id = prior_ids[(int64_t)b * prior_stride + j];
                if (prior_cnt[(int64_t)b * prior_stride + j] >= 1 && id >= 0 && id < V) listed[id] = 1;
            }
        if (q.flags & OF_BIAS)
            for (int j = 0; j < q.n_bias; ++j) {
                int id = bias_ids[(int64_t)b * bias_stride + j];
                if (id >= 0 && id < V) listed[id] = 1;
            }
        for (int t = 0; t < Zv; ++t) {
            int lo = t * tile, hi = lo + tile < V ? lo + tile : V;
            int cnt = 0;
            for (int i = lo; i < hi; ++i)
                if (!listed[i]) { work[cnt].z = z[i]; work[cnt].id = i; ++cnt; }
            qsort(work, (size_t)cnt, sizeof(zid), zid_cmp);
            int32_t* o = out_ids + ((int64_t)r * Zv + t) * OK_MAX;
            for (int k = 0; k < OK_MAX; ++k) o[k] = k < cnt ? work[k].id : -1;
        }
    }
    free(z); free(work); free(listed);
    return 0;
}

/* Array forms of the spec functions, for the tests' sweeps. */
void oracle_exp_spec_n(const float* x, float* y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) y[i] = oracle_exp_spec(x[i]);
}

void oracle_log_spec_n(const float* x, float* y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) y[i] = oracle_log_spec(x[i]);
}

/* ======================================================================
 * Whole-domain sweeps of the spec functions, for the tests: element i of
 * a range takes the 32-bit pattern first + i as its argument.
 *   fn 0: oracle_exp_spec          (argument: float bits)
 *   fn 1: oracle_log_spec          (argument: float bits)
 *   fn 2: Gumbel noise -ln(-ln u) of the uniform u of the Philox words
 *         whose top 23 bits are the argument               (argument < 2^23)
 *   fn 3: Philox word for counter (first + i, c1, c2)    (seed, offset)
 *   fn 4: Gumbel noise for counter (first + i, c1, c2)   (seed, offset)
 * Results are written as 32-bit patterns.
 * ====================================================================== */
typedef struct {
    int fn;
    uint32_t first, c1, c2;
    uint64_t seed, offset;
    uint32_t* out;
    int64_t lo, hi;
} sweep_job;

static uint32_t sweep_one(const sweep_job* j, uint32_t a)
{
    switch (j->fn) {
    case 0: return f2u(oracle_exp_spec(u2f(a)));
    case 1: return f2u(oracle_log_spec(u2f(a)));
    case 2: return f2u(-oracle_log_spec(-oracle_log_spec(oracle_uniform(a << 9))));
    case 3: return oracle_philox_word(j->seed, j->offset, a, j->c1, j->c2);
    default: return f2u(oracle_gumbel(j->seed, j->offset, a, j->c1, j->c2));
    }
}

static void* sweep_worker(void* p)
{
    sweep_job* j = (sweep_job*)p;
    for (int64_t i = j->lo; i < j->hi; ++i) j->out[i] = sweep_one(j, j->first + (uint32_t)i);
    return NULL;
}

int oracle_spec_sweep(int fn, uint32_t first, int64_t n, uint32_t c1, uint32_t c2, uint64_t seed,
                      uint64_t offset, uint32_t* out, int threads)
{
    if (fn < 0 || fn > 4 || n < 0) return -1;
    if (threads < 1) threads = 1;
    if (threads > 64) threads = 64;
    sweep_job jobs[64];
    pthread_t tid[64];
    for (int t = 0; t < threads; ++t) {
        sweep_job j = {fn, first, c1, c2, seed, offset, out, n * t / threads, n * (t + 1) / threads};
        jobs[t] = j;
        if (threads == 1) sweep_worker(&jobs[t]);
        else pthread_create(&tid[t], NULL, sweep_worker, &jobs[t]);
    }
    if (threads > 1)
        for (int t = 0; t < threads; ++t) pthread_join(tid[t], NULL);
    return 0;
}
