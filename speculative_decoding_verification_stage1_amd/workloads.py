"""Seeded synthetic inputs for the sampling, verification and top-k workloads.

This module only draws random inputs (logits, per-request settings, penalty
and bias lists, grammar bitmasks, draft distributions and draft tokens).  It
holds none of the sampler's arithmetic, so the CPU oracle and the HIP path can
both be fed from it.  Every array is produced by numpy's PCG64 generator from
an explicit seed.

Shapes and value distributions follow the workloads stated for the method:

* ``c0``  B=1, V=2^15 fp32, logits 2*N(0,1) plus +10 on 8 random ids,
  T=0.8, top-k 128, top-p 0.9, min-p 0, no penalties or grammar; one greedy
  and one stochastic request.
* ``c1``  B=64, V=2^17 bf16, mixed per-request settings (half greedy,
  T~U[0.5,1.5], top-k in {off,50,128}, top-p in {1,0.9,0.95}, min-p in
  {0,0.05}), repetition penalty 1.1 over 64 prior ids with counts U{1..5},
  frequency 0.2 / presence 0.1, 16 logit-bias entries in U[-5,5].
* ``c2``  B=256, V=2^18 bf16, everything of c1 plus a packed uint32 grammar
  bitmask with 5% of tokens allowed and one of the raw top-10 forced allowed.
* ``c3``  speculative verification: B=64, gamma=4, V=2^17, target logits
  (B*5)xV bf16, draft probabilities softmax(target + N(0,0.5)) as B x 4 x V
  fp32, draft ids drawn from them, a quarter of the requests greedy.
* ``c4``  top-k stress: B=512, V=2^18 fp32, k=128, peaked (as c0) or flat
  N(0,0.1) logits.

"N(0,s)" means a normal with standard deviation s.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

DTYPE_F32 = 0
DTYPE_BF16 = 1

PRIOR_LEN = 64   # prior-token list length used by the workloads
BIAS_LEN = 16    # logit-bias list length used by the workloads


def data_seed(config: int) -> int:
    """Seed of the data generator for workload ``c<config>``."""
    return 1000 + config


@dataclasses.dataclass
class Requests:
    """Per-request sampling settings, one entry per request (row)."""
    greedy: np.ndarray        # bool [B]
    temperature: np.ndarray   # f32  [B]
    top_k: np.ndarray         # i32  [B]; 0 means top-k off
    top_p: np.ndarray         # f32  [B]; 1.0 means top-p off
    min_p: np.ndarray         # f32  [B]; 0.0 means min-p off
    rep_penalty: np.ndarray   # f32  [B]; 1.0 means off
    freq_penalty: np.ndarray  # f32  [B]
    pres_penalty: np.ndarray  # f32  [B]
    use_penalties: np.ndarray  # bool [B]; prior list applies
    use_bias: np.ndarray      # bool [B]
    use_grammar: np.ndarray   # bool [B]
    prior_ids: np.ndarray     # i32 [B, P]
    prior_cnt: np.ndarray     # i32 [B, P]
    n_prior: np.ndarray       # i32 [B]
    bias_ids: np.ndarray      # i32 [B, NB]
    bias_val: np.ndarray      # f32 [B, NB]
    n_bias: np.ndarray        # i32 [B]
    bitmask: Optional[np.ndarray] = None  # u32 [B, ceil(V/32)] or None

    @property
    def batch(self) -> int:
        return int(self.greedy.shape[0])


def plain_requests(B: int, *, greedy=False, temperature=1.0, top_k=0, top_p=1.0,
                   min_p=0.0, prior_len: int = 1, bias_len: int = 1) -> Requests:
    """Requests with the same settings everywhere and no lists or grammar."""
    return Requests(
        greedy=np.full(B, bool(greedy)),
        temperature=np.full(B, temperature, np.float32),
        top_k=np.full(B, top_k, np.int32),
        top_p=np.full(B, top_p, np.float32),
        min_p=np.full(B, min_p, np.float32),
        rep_penalty=np.ones(B, np.float32),
        freq_penalty=np.zeros(B, np.float32),
        pres_penalty=np.zeros(B, np.float32),
        use_penalties=np.zeros(B, bool),
        use_bias=np.zeros(B, bool),
        use_grammar=np.zeros(B, bool),
        prior_ids=np.full((B, prior_len), -1, np.int32),
        prior_cnt=np.zeros((B, prior_len), np.int32),
        n_prior=np.zeros(B, np.int32),
        bias_ids=np.full((B, bias_len), -1, np.int32),
        bias_val=np.zeros((B, bias_len), np.float32),
        n_bias=np.zeros(B, np.int32),
        bitmask=None,
    )


# ----------------------------------------------------------------------------
# logits
# ----------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round to nearest even); return the raw
    16-bit patterns as uint16."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen raw bfloat16 patterns to fp32 (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def peaked_logits(rng: np.random.Generator, rows: int, V: int, n_peaks: int = 8,
                  scale: float = 2.0, boost: float = 10.0) -> np.ndarray:
    """fp32 [rows, V]: scale*N(0,1) plus ``boost`` on ``n_peaks`` distinct
    random ids per row (a peaked, low-entropy next-token distribution)."""
    x = rng.standard_normal((rows, V), dtype=np.float32)
    x *= np.float32(scale)
    k = min(n_peaks, V)
    for r in range(rows):
        ids = rng.choice(V, size=k, replace=False)
        x[r, ids] += np.float32(boost)
    return x


def flat_logits(rng: np.random.Generator, rows: int, V: int, std: float = 0.1) -> np.ndarray:
    x = rng.standard_normal((rows, V), dtype=np.float32)
    x *= np.float32(std)
    return x


# ----------------------------------------------------------------------------
# per-request settings and side lists
# ----------------------------------------------------------------------------

def mixed_requests(rng: np.random.Generator, B: int, V: int, *, penalties: bool = True,
                   bias: bool = True, prior_len: int = PRIOR_LEN,
                   bias_len: int = BIAS_LEN) -> Requests:
    """The heterogeneous batch: exactly floor(B/2) greedy rows (seeded
    permutation), T~U[0.5,1.5], top-k in {off,50,128}, top-p in
    {1.0,0.9,0.95}, min-p in {0,0.05}; repetition 1.1 / frequency 0.2 /
    presence 0.1 over ``prior_len`` distinct prior ids with counts U{1..5};
    ``bias_len`` distinct logit-bias ids with values U[-5,5]."""
    greedy = np.zeros(B, bool)
    greedy[rng.permutation(B)[: B // 2]] = True
    temperature = rng.uniform(0.5, 1.5, B).astype(np.float32)
    top_k = rng.choice(np.array([0, 50, 128], np.int32), B).astype(np.int32)
    top_p = rng.choice(np.array([1.0, 0.9, 0.95], np.float32), B).astype(np.float32)
    min_p = rng.choice(np.array([0.0, 0.05], np.float32), B).astype(np.float32)
    P = prior_len
    NB = bias_len
    prior_ids = np.full((B, P), -1, np.int32)
    prior_cnt = np.zeros((B, P), np.int32)
    bias_ids = np.full((B, NB), -1, np.int32)
    bias_val = np.zeros((B, NB), np.float32)
    n_prior = np.zeros(B, np.int32)
    n_bias = np.zeros(B, np.int32)
    for r in range(B):
        if penalties:
            k = min(P, V)
            prior_ids[r, :k] = rng.choice(V, size=k, replace=False)
            prior_cnt[r, :k] = rng.integers(1, 6, size=k)
            n_prior[r] = k
        if bias:
            k = min(NB, V)
            bias_ids[r, :k] = rng.choice(V, size=k, replace=False)
            bias_val[r, :k] = rng.uniform(-5.0, 5.0, size=k).astype(np.float32)
            n_bias[r] = k
    return Requests(
        greedy=greedy, temperature=temperature, top_k=top_k, top_p=top_p, min_p=min_p,
        rep_penalty=np.full(B, 1.1 if penalties else 1.0, np.float32),
        freq_penalty=np.full(B, 0.2 if penalties else 0.0, np.float32),
        pres_penalty=np.full(B, 0.1 if penalties else 0.0, np.float32),
        use_penalties=np.full(B, bool(penalties)),
        use_bias=np.full(B, bool(bias)),
        use_grammar=np.zeros(B, bool),
        prior_ids=prior_ids, prior_cnt=prior_cnt, n_prior=n_prior,
        bias_ids=bias_ids, bias_val=bias_val, n_bias=n_bias,
    )


def grammar_bitmask(rng: np.random.Generator, raw_logits: np.ndarray,
                    allowed_frac: float = 0.05, force_topn: int = 10) -> np.ndarray:
    """Packed grammar bitmask, uint32 [B, ceil(V/32)], bit (i & 31) of word
    (i >> 5) set when token i is allowed.  Bits are i.i.d. Bernoulli
    (``allowed_frac``); one id drawn uniformly from each row's raw top-
    ``force_topn`` logits is forced allowed."""
    B, V = raw_logits.shape
    W = (V + 31) // 32
    out = np.zeros((B, W), np.uint32)
    for r in range(B):
        allowed = rng.random(V, dtype=np.float32) < np.float32(allowed_frac)
        n = min(force_topn, V)
        top = np.argpartition(-raw_logits[r], n - 1)[:n]
        allowed[rng.choice(top)] = True
        padded = np.zeros(W * 32, bool)
        padded[:V] = allowed
        out[r] = np.packbits(padded, bitorder="little").view("<u4")
    return out


# ----------------------------------------------------------------------------
# the named workloads
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class SampleWorkload:
    name: str
    dtype: int               # DTYPE_F32 or DTYPE_BF16
    logits: np.ndarray       # f32 [B, V] or u16 (bf16 bits) [B, V]
    req: Requests
    seed: int = 0            # Philox seed
    offset: int = 0          # Philox offset

    @property
    def B(self) -> int:
        return int(self.logits.shape[0])

    @property
    def V(self) -> int:
        return int(self.logits.shape[1])


def workload_c0(greedy: bool) -> SampleWorkload:
    rng = np.random.default_rng(data_seed(0))
    x = peaked_logits(rng, 1, 32768)
    req = plain_requests(1, greedy=greedy, temperature=0.8, top_k=128, top_p=0.9, min_p=0.0)
    return SampleWorkload("c0-greedy" if greedy else "c0-stochastic", DTYPE_F32, x, req)


def workload_mixed(config: int, B: int, V: int, grammar: bool, rows: Optional[int] = None) -> SampleWorkload:
    """c1 (grammar=False) or c2 (grammar=True) style batch.  ``rows`` limits
    the number of rows actually generated (the first ``rows`` of the
    sequence) for tests that only need a few."""
    rng = np.random.default_rng(data_seed(config))
    n = B if rows is None else rows
    raw = peaked_logits(rng, n, V)
    req = mixed_requests(rng, n, V)
    if grammar:
        req.bitmask = grammar_bitmask(rng, raw)
        req.use_grammar = np.ones(n, bool)
    name = f"c{config}"
    return SampleWorkload(name, DTYPE_BF16, to_bf16_bits(raw), req)


def workload_c1(rows: Optional[int] = None) -> SampleWorkload:
    return workload_mixed(1, 64, 131072, grammar=False, rows=rows)


def workload_c2(rows: Optional[int] = None) -> SampleWorkload:
    return workload_mixed(2, 256, 262144, grammar=True, rows=rows)


STRESS_KINDS = ("logprob", "sparse_grammar", "listed_tile", "listed_100")


def workload_c2_stress(kind: str, rows: Optional[int] = None, B: int = 256, V: int = 262144) -> SampleWorkload:
    """c2's batch (B=256, V=2^18 bf16, the same per-request settings) with
    one thing changed, to exercise the tile stage off its usual path:

    * ``logprob``: every row replaced by its log-softmax (float64
      log-sum-exp, rounded to fp32 then bf16), so that every logit is
      negative, as when the sampler is fed log-probabilities;
    * ``sparse_grammar``: grammar bitmask with 0.1 % of the tokens allowed
      (Bernoulli(0.001), one of the raw top-10 forced allowed): about 33
      allowed tokens per 32768-token tile;
    * ``listed_tile``: no grammar; each request's prior list holds 200
      distinct ids drawn from [0, 32768) with counts U{1..5} (plus the 16
      bias ids anywhere), so one vocabulary tile holds more than 128 tokens
      named by the lists;
    * ``listed_100``: the same with 100 prior ids, so that one tile holds
      about 100 listed tokens (fewer than 128).
    """
    if kind not in STRESS_KINDS:
        raise ValueError(kind)
    n = B if rows is None else rows
    rng = np.random.default_rng(data_seed(2))
    raw = peaked_logits(rng, n, V)
    req = mixed_requests(rng, n, V)
    req.bitmask = grammar_bitmask(rng, raw)
    req.use_grammar = np.ones(n, bool)
    rs = np.random.default_rng(data_seed(2) + 100 + STRESS_KINDS.index(kind))
    if kind == "logprob":
        x = raw.astype(np.float64)
        m = x.max(axis=1, keepdims=True)
        lse = m + np.log(np.exp(x - m).sum(axis=1, keepdims=True))
        raw = (x - lse).astype(np.float32)
    elif kind == "sparse_grammar":
        req.bitmask = grammar_bitmask(rs, raw, allowed_frac=0.001)
    else:
        req.bitmask = None
        req.use_grammar = np.zeros(n, bool)
        P = 200 if kind == "listed_tile" else 100
        req.prior_ids = np.full((n, P), -1, np.int32)
        req.prior_cnt = np.zeros((n, P), np.int32)
        for r in range(n):
            req.prior_ids[r] = rs.choice(min(32768, V), size=P, replace=False)
            req.prior_cnt[r] = rs.integers(1, 6, size=P)
        req.n_prior = np.full(n, P, np.int32)
    return SampleWorkload(f"c2-{kind}", DTYPE_BF16, to_bf16_bits(raw), req)


@dataclasses.dataclass
class VerifyWorkload:
    name: str
    dtype: int
    target: np.ndarray       # bf16 bits u16 [B*(gamma+1), V] or f32
    draft_probs: np.ndarray  # f32 [B, gamma, V]
    draft_ids: np.ndarray    # i32 [B, gamma]
    req: Requests            # one entry per request
    gamma: int
    seed: int = 0
    offset: int = 0

    @property
    def B(self) -> int:
        return int(self.draft_ids.shape[0])

    @property
    def V(self) -> int:
        return int(self.target.shape[1])


def draft_distribution(rng: np.random.Generator, target_f32: np.ndarray, noise_std: float) -> np.ndarray:
    """Draft model stand-in: softmax(target + N(0, noise_std)) in float64,
    stored as fp32."""
    y = target_f32.astype(np.float64) + rng.standard_normal(target_f32.shape) * noise_std
    y -= y.max(axis=-1, keepdims=True)
    np.exp(y, out=y)
    y /= y.sum(axis=-1, keepdims=True)
    return y.astype(np.float32)


def draw_from(rng: np.random.Generator, probs_f32: np.ndarray) -> int:
    """One categorical draw from a probability row (float64 inverse CDF)."""
    c = np.cumsum(probs_f32.astype(np.float64))
    u = rng.random() * c[-1]
    return int(min(np.searchsorted(c, u, side="right"), len(c) - 1))


def workload_verify(B: int = 64, gamma: int = 4, V: int = 131072, config: int = 3,
                    greedy_frac: float = 0.25, noise_std: float = 0.5) -> VerifyWorkload:
    """c3: target logits as c0 (one independent row per (request, position)),
    draft probabilities softmax(target + N(0, noise_std)) for the gamma draft
    positions, draft ids drawn from those, floor(B*greedy_frac) greedy
    requests; stochastic requests use T=1 with no top-k/top-p/min-p."""
    rng = np.random.default_rng(data_seed(config))
    rows = B * (gamma + 1)
    raw = peaked_logits(rng, rows, V)
    bits = to_bf16_bits(raw)
    tgt = bf16_bits_to_f32(bits).reshape(B, gamma + 1, V)
    q = np.empty((B, gamma, V), np.float32)
    d = np.empty((B, gamma), np.int32)
    for b in range(B):
        q[b] = draft_distribution(rng, tgt[b, :gamma], noise_std)
        for j in range(gamma):
            d[b, j] = draw_from(rng, q[b, j])
    req = plain_requests(B, temperature=1.0)
    g = np.zeros(B, bool)
    g[rng.permutation(B)[: int(B * greedy_frac)]] = True
    req.greedy = g
    return VerifyWorkload("c3", DTYPE_BF16, bits, q, d, req, gamma)


@dataclasses.dataclass
class TopkWorkload:
    name: str
    dtype: int
    logits: np.ndarray
    k: int


def workload_c4(regime: str, rows: Optional[int] = None, B: int = 512, V: int = 262144) -> TopkWorkload:
    """c4: fp32 [B, V], ``regime`` 'peaked' (as c0) or 'flat' (N(0,0.1))."""
    rng = np.random.default_rng(data_seed(4) + (0 if regime == "peaked" else 1))
    n = B if rows is None else rows
    if regime == "peaked":
        x = peaked_logits(rng, n, V)
    elif regime == "flat":
        x = flat_logits(rng, n, V)
    else:
        raise ValueError(regime)
    return TopkWorkload(f"c4-{regime}", DTYPE_F32, x, 128)


# ----------------------------------------------------------------------------
# LM head (hidden states and vocabulary weights)
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class LmheadWorkload:
    name: str
    hidden: np.ndarray   # uint16 [B, D] bf16 patterns
    weight: np.ndarray   # uint16 [V, D] bf16 patterns, one row per token
    req: Requests
    exact: bool          # every product and partial sum exact in binary32


LMHEAD_KINDS = ("normal", "grid")


def workload_lmhead(kind: str = "normal", B: int = 64, D: int = 4096, V: int = 131072,
                    seed: Optional[int] = None) -> LmheadWorkload:
    """Synthetic LM head (seed data_seed(5) unless given).
    'normal': weight ~ N(0, (2/sqrt(D))^2), hidden ~ N(0, 1), so logits have
    a standard deviation of about 2; every second row also has a few
    (2..8) tokens lifted by adding 4/|w_t|^2 * w_t per token to the hidden
    state (about +4 on those logits), a peaked distribution.
    'grid': hidden in {-1, -7/8, .., 1} and weights in {-1, -63/64, .., 1}
    (uniform), so every product is a multiple of 2^-9 and every partial sum
    stays below 2^12 in magnitude: the logits are exact in binary32 for any
    summation order (D <= 4096), with many exact ties.
    Requests: mixed_requests without lists (greedy half, T, top-k, top-p,
    min-p mixes)."""
    rng = np.random.default_rng(data_seed(5) if seed is None else seed)
    req = mixed_requests(rng, B, V, penalties=False, bias=False)
    if kind == "grid":
        if D > 4096:
            raise ValueError("grid inputs are exact only up to D = 4096")
        h = to_bf16_bits((rng.integers(-8, 9, (B, D)) / 8).astype(np.float32))
        w = to_bf16_bits((rng.integers(-64, 65, (V, D), dtype=np.int16) / np.float32(64)).astype(np.float32))
        return LmheadWorkload(f"lmhead-grid-{B}x{D}x{V}", h, w, req, True)
    if kind != "normal":
        raise ValueError(kind)
    wf = np.empty((V, D), np.float32)
    step = max(1, (1 << 24) // D)
    for v0 in range(0, V, step):   # in slices, to bound the float64 temporaries
        wf[v0:v0 + step] = rng.standard_normal((min(step, V - v0), D), dtype=np.float32) * np.float32(2 / np.sqrt(D))
    w = to_bf16_bits(wf)
    wf = bf16_bits_to_f32(w)
    hf = rng.standard_normal((B, D), dtype=np.float32)
    for b in range(1, B, 2):
        for t in rng.choice(V, int(rng.integers(2, 9)), replace=False):
            hf[b] += np.float32(4.0 / float(np.dot(wf[t], wf[t]))) * wf[t]
    del wf
    return LmheadWorkload(f"lmhead-normal-{B}x{D}x{V}", to_bf16_bits(hf), w, req, False)


def lmhead_device_inputs(B: int, D: int, V: int, seed: Optional[int] = None, device="cuda"):
    """The 'normal' LM-head recipe of workload_lmhead drawn on the device
    with torch's seeded generator (fast at vocabulary scale; not the same
    values as the host recipe): bf16 hidden [B, D] and weight [V, D] and the
    host requests."""
    import torch
    s = data_seed(5) if seed is None else seed
    rng = np.random.default_rng(s)
    req = mixed_requests(rng, B, V, penalties=False, bias=False)
    g = torch.Generator(device=device)
    g.manual_seed(s)
    w = torch.empty((V, D), dtype=torch.bfloat16, device=device)
    step = max(1, (1 << 26) // D)
    for v0 in range(0, V, step):
        n = min(step, V - v0)
        w[v0:v0 + n] = (torch.randn((n, D), generator=g, device=device) * (2.0 / D ** 0.5)).to(torch.bfloat16)
    h = torch.randn((B, D), generator=g, device=device)
    for b in range(1, B, 2):
        for t in rng.choice(V, int(rng.integers(2, 9)), replace=False):
            wt = w[int(t)].float()
            h[b] += (4.0 / float(torch.dot(wt, wt))) * wt
    return h.to(torch.bfloat16), w, req
