"""ctypes binding of the CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``.  The product library never loads
it.  The oracle is a plain, slow statement of the sampler; see the header of
``oracle.c`` for the definitions it follows and ``tests/test_oracle_*.py``
for the pins that tie it to the pages and to independent references.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FLAG_GREEDY = 1 << 0
FLAG_GRAMMAR = 1 << 1
FLAG_REP = 1 << 2
FLAG_FREQPRES = 1 << 3
FLAG_BIAS = 1 << 4
FLAG_TOPK = 1 << 5
FLAG_TOPP = 1 << 6
FLAG_MINP = 1 << 7
FLAG_DRAFT_HIST = 1 << 8   # verification: earlier drafts join the penalty history

KMAX = 128

STATUS_OK = 0
STATUS_ALL_MASKED = 1
STATUS_INVALID = 2
STATUS_TOPK_CLAMPED = 3

OREQ = np.dtype([
    ("flags", "<u4"), ("temperature", "<f4"), ("top_k", "<i4"), ("top_p", "<f4"),
    ("min_p", "<f4"), ("rep", "<f4"), ("freq", "<f4"), ("pres", "<f4"),
    ("n_prior", "<i4"), ("n_bias", "<i4"),
])


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (plain C99, no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
               "-shared", "-pthread", "-o", _LIB, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, u64 = ctypes.c_int, ctypes.c_int64, ctypes.c_uint64
        L.oracle_philox4x32_10.argtypes = [P, P, P]
        L.oracle_exp_spec.argtypes = [ctypes.c_float]
        L.oracle_exp_spec.restype = ctypes.c_float
        L.oracle_log_spec.argtypes = [ctypes.c_float]
        L.oracle_log_spec.restype = ctypes.c_float
        L.oracle_exp_spec_n.argtypes = [P, P, i64]
        L.oracle_log_spec_n.argtypes = [P, P, i64]
        L.oracle_spec_sweep.argtypes = [i32, ctypes.c_uint32, i64, ctypes.c_uint32, ctypes.c_uint32, u64, u64, P,
                                        i32]
        L.oracle_spec_sweep.restype = i32
        L.oracle_uniform.argtypes = [ctypes.c_uint32]
        L.oracle_uniform.restype = ctypes.c_float
        L.oracle_philox_word.argtypes = [u64, u64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
        L.oracle_philox_word.restype = ctypes.c_uint32
        L.oracle_gumbel.argtypes = [u64, u64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
        L.oracle_gumbel.restype = ctypes.c_float
        L.oracle_prelude_row.argtypes = [P, i32, i32, ctypes.c_uint32, P, P, P, i32, P, P, i32,
                                         ctypes.c_float, ctypes.c_float, ctypes.c_float, P]
        L.oracle_sample.argtypes = [P, i32, i32, i32, i64, P, P, P, i32, P, P, i32, P, i64,
                                    u64, u64, P, P, P, P, P, P, i32]
        L.oracle_sample.restype = i32
        L.oracle_verify.argtypes = [P, i32, i32, i32, i32, i64, P, P, P, i32, P, P, i32, P, i64,
                                    P, P, P, u64, u64, P, P, P, i32]
        L.oracle_verify.restype = i32
        L.oracle_verify_dense.argtypes = [P, i32, i32, i32, i32, i64, P, P, P, P, u64, u64,
                                          ctypes.c_double, P, P, P, P, i32]
        L.oracle_verify_dense.restype = i32
        L.oracle_topk.argtypes = [P, i32, i32, i32, i64, i32, P, P, i32]
        L.oracle_topk.restype = i32
        L.oracle_tile_topk.argtypes = [P, i32, i32, i32, i64, i32, i32, P, P, P, i32, P, P, i32,
                                       P, i64, P]
        L.oracle_tile_topk.restype = i32
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------------
# scalar helpers
# ---------------------------------------------------------------------------

def philox(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    lib().oracle_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def exp_spec(x: float) -> np.float32:
    return np.float32(lib().oracle_exp_spec(float(np.float32(x))))


def log_spec(x: float) -> np.float32:
    return np.float32(lib().oracle_log_spec(float(np.float32(x))))


def exp_spec_n(x) -> np.ndarray:
    a = np.ascontiguousarray(x, np.float32)
    y = np.empty_like(a)
    lib().oracle_exp_spec_n(_p(a), _p(y), a.size)
    return y


def log_spec_n(x) -> np.ndarray:
    a = np.ascontiguousarray(x, np.float32)
    y = np.empty_like(a)
    lib().oracle_log_spec_n(_p(a), _p(y), a.size)
    return y


def uniform(w: int) -> np.float32:
    return np.float32(lib().oracle_uniform(int(w)))


SWEEP_EXP, SWEEP_LOG, SWEEP_GUMBEL_WORD, SWEEP_PHILOX, SWEEP_GUMBEL = range(5)


def spec_sweep(fn: int, first: int, n: int, c1: int = 0, c2: int = 0, seed: int = 0, offset: int = 0,
               threads: int = 1) -> np.ndarray:
    """32-bit results of a spec function over the arguments first .. first
    + n - 1 (float bit patterns, Philox words, or counter words c0; see
    oracle_spec_sweep)."""
    out = np.empty(n, np.uint32)
    rc = lib().oracle_spec_sweep(fn, first & 0xFFFFFFFF, n, c1, c2, seed, offset, _p(out), threads)
    assert rc == 0
    return out


def philox_word(seed: int, offset: int, c0: int, c1: int, c2: int) -> int:
    return int(lib().oracle_philox_word(seed, offset, c0, c1, c2))


def gumbel(seed: int, offset: int, c0: int, c1: int, c2: int) -> np.float32:
    return np.float32(lib().oracle_gumbel(seed, offset, c0, c1, c2))


# ---------------------------------------------------------------------------
# requests
# ---------------------------------------------------------------------------

def flags_of(req, i: int) -> int:
    f = 0
    if req.greedy[i]:
        f |= FLAG_GREEDY
    if req.use_grammar[i]:
        f |= FLAG_GRAMMAR
    if req.use_penalties[i]:
        f |= FLAG_REP | FLAG_FREQPRES
    if req.use_bias[i]:
        f |= FLAG_BIAS
    if req.top_k[i] > 0:
        f |= FLAG_TOPK
    if req.top_p[i] < 1.0:
        f |= FLAG_TOPP
    if req.min_p[i] > 0.0:
        f |= FLAG_MINP
    return f


def pack_requests(req, flags=None) -> np.ndarray:
    B = req.batch
    a = np.zeros(B, OREQ)
    for i in range(B):
        a[i]["flags"] = flags_of(req, i) if flags is None else flags[i]
    a["temperature"] = req.temperature
    a["top_k"] = req.top_k
    a["top_p"] = req.top_p
    a["min_p"] = req.min_p
    a["rep"] = req.rep_penalty
    a["freq"] = req.freq_penalty
    a["pres"] = req.pres_penalty
    a["n_prior"] = req.n_prior
    a["n_bias"] = req.n_bias
    return a


def _lists(req):
    pid = np.ascontiguousarray(req.prior_ids, np.int32)
    pc = np.ascontiguousarray(req.prior_cnt, np.int32)
    bid = np.ascontiguousarray(req.bias_ids, np.int32)
    bv = np.ascontiguousarray(req.bias_val, np.float32)
    bm = None if req.bitmask is None else np.ascontiguousarray(req.bitmask, np.uint32)
    return pid, pc, bid, bv, bm


def prelude_row(logits_row, dtype: int, flags: int, req, b: int, bitmask_row=None) -> np.ndarray:
    """Processed logits z for one row (request b's lists)."""
    x = np.ascontiguousarray(logits_row)
    V = x.shape[-1]
    z = np.zeros(V, np.float32)
    pid, pc, bid, bv, bm = _lists(req)
    bmr = None
    if bitmask_row is not None:
        bmr = np.ascontiguousarray(bitmask_row, np.uint32)
    elif bm is not None:
        bmr = np.ascontiguousarray(bm[b])
    lib().oracle_prelude_row(
        _p(x), dtype, V, flags, _p(bmr),
        _p(np.ascontiguousarray(pid[b])), _p(np.ascontiguousarray(pc[b])), int(req.n_prior[b]),
        _p(np.ascontiguousarray(bid[b])), _p(np.ascontiguousarray(bv[b])), int(req.n_bias[b]),
        float(req.rep_penalty[b]), float(req.freq_penalty[b]), float(req.pres_penalty[b]), _p(z))
    return z


def sample(logits, dtype: int, req, seed: int = 0, offset: int = 0, threads: int = 1,
           flags=None, packed=None):
    """Batched single-step sampling.  Returns a dict with tokens [B],
    topk_ids [B,128], probs [B,128], kept [B], mass [B], status [B]."""
    x = np.ascontiguousarray(logits)
    B, V = x.shape
    r = pack_requests(req, flags) if packed is None else packed
    pid, pc, bid, bv, bm = _lists(req)
    out = dict(tokens=np.zeros(B, np.int32), topk_ids=np.zeros((B, KMAX), np.int32),
               probs=np.zeros((B, KMAX), np.float32), kept=np.zeros(B, np.int32),
               mass=np.zeros(B, np.float32), status=np.zeros(B, np.int32))
    rc = lib().oracle_sample(
        _p(x), dtype, B, V, V, _p(r), _p(pid), _p(pc), pid.shape[1], _p(bid), _p(bv), bid.shape[1],
        _p(bm), 0 if bm is None else bm.shape[1], seed, offset,
        _p(out["tokens"]), _p(out["topk_ids"]), _p(out["probs"]), _p(out["kept"]),
        _p(out["mass"]), _p(out["status"]), threads)
    if rc != 0:
        raise ValueError("oracle_sample rejected its arguments")
    return out


def verify(target, dtype: int, B: int, gamma: int, req, draft_ids, draft_probs, bitmask=None,
           seed: int = 0, offset: int = 0, threads: int = 1, flags=None, packed=None, cu_num_draft=None):
    """Speculative verification of gamma drafts for B requests (or of
    n_b = cu[b] - cu[b-1] <= gamma drafts each, with the inclusive cumulative
    counts `cu_num_draft`; tensors keep their gamma-wide layout).  Returns a
    dict with tokens [B, gamma+1] (-1 padded), n_emit [B], status [B]."""
    x = np.ascontiguousarray(target)
    rows, V = x.shape
    assert rows == B * (gamma + 1)
    r = pack_requests(req, flags) if packed is None else packed
    pid, pc, bid, bv, _ = _lists(req)
    bm = None if bitmask is None else np.ascontiguousarray(bitmask, np.uint32)
    d = np.ascontiguousarray(draft_ids, np.int32)
    q = np.ascontiguousarray(draft_probs, np.float32)
    cu = None if cu_num_draft is None else np.ascontiguousarray(cu_num_draft, np.int32)
    assert cu is None or cu.shape == (B,)
    out = dict(tokens=np.zeros((B, gamma + 1), np.int32), n_emit=np.zeros(B, np.int32),
               status=np.zeros(B, np.int32))
    rc = lib().oracle_verify(
        _p(x), dtype, B, gamma, V, V, _p(r), _p(pid), _p(pc), pid.shape[1], _p(bid), _p(bv),
        bid.shape[1], _p(bm), 0 if bm is None else bm.shape[1], _p(d), _p(q), _p(cu), seed, offset,
        _p(out["tokens"]), _p(out["n_emit"]), _p(out["status"]), threads)
    if rc != 0:
        raise ValueError("oracle_verify rejected its arguments")
    return out


def verify_dense(target, dtype: int, B: int, gamma: int, req, draft_ids, draft_probs=None, seed: int = 0,
                 offset: int = 0, threads: int = 1, flags=None, packed=None, cu_num_draft=None,
                 zslack: float = 1e-5):
    """Dense verification (full-vocabulary p; draft_probs None: no draft
    probabilities).  Returns tokens [B, gamma+1] (-1 padded), n_emit [B],
    status [B] and fragile [B] (1 where the tokens depend on Z to within a
    relative `zslack`)."""
    x = np.ascontiguousarray(target)
    rows, V = x.shape
    assert rows == B * (gamma + 1)
    r = pack_requests(req, flags) if packed is None else packed
    d = np.ascontiguousarray(draft_ids, np.int32)
    q = None if draft_probs is None else np.ascontiguousarray(draft_probs, np.float32)
    cu = None if cu_num_draft is None else np.ascontiguousarray(cu_num_draft, np.int32)
    assert cu is None or cu.shape == (B,)
    out = dict(tokens=np.zeros((B, gamma + 1), np.int32), n_emit=np.zeros(B, np.int32),
               status=np.zeros(B, np.int32), fragile=np.zeros(B, np.int32))
    rc = lib().oracle_verify_dense(
        _p(x), dtype, B, gamma, V, V, _p(r), _p(d), _p(q), _p(cu), seed, offset, zslack,
        _p(out["tokens"]), _p(out["n_emit"]), _p(out["status"]), _p(out["fragile"]), threads)
    if rc != 0:
        raise ValueError("oracle_verify_dense rejected its arguments")
    return out


def topk(logits, dtype: int, k: int, threads: int = 1):
    x = np.ascontiguousarray(logits)
    B, V = x.shape
    ids = np.zeros((B, k), np.int32)
    vals = np.zeros((B, k), np.float32)
    rc = lib().oracle_topk(_p(x), dtype, B, V, V, k, _p(ids), _p(vals), threads)
    if rc != 0:
        raise ValueError("oracle_topk rejected its arguments")
    return ids, vals


def tile_topk(logits, dtype: int, tile: int, req=None, rows_per_req: int = 1, bitmask=None,
              flags=None):
    """First 128 ids of every vocabulary tile (listed ids left out)."""
    x = np.ascontiguousarray(logits)
    rows, V = x.shape
    Zv = (V + tile - 1) // tile
    out = np.zeros((rows, Zv, KMAX), np.int32)
    if req is None:
        rc = lib().oracle_tile_topk(_p(x), dtype, rows, V, V, tile, rows_per_req, None,
                                    None, None, 0, None, None, 0, None, 0, _p(out))
    else:
        r = pack_requests(req, flags)
        pid, pc, bid, bv, bm0 = _lists(req)
        bm = bm0 if bitmask is None else np.ascontiguousarray(bitmask, np.uint32)
        rc = lib().oracle_tile_topk(_p(x), dtype, rows, V, V, tile, rows_per_req, _p(r),
                                    _p(pid), _p(pc), pid.shape[1], _p(bid), _p(bv), bid.shape[1],
                                    _p(bm), 0 if bm is None else bm.shape[1], _p(out))
    if rc != 0:
        raise ValueError("oracle_tile_topk rejected its arguments")
    return out


# ---------------------------------------------------------------------------
# LM head (the fused projection + sampling variant)
# ---------------------------------------------------------------------------

def _widen_bf16(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def lmhead_logits(hidden_bits, weight_bits) -> np.ndarray:
    """LM-head logits z = H W^T in float64 from raw bf16 patterns: hidden
    [B, D], weight [V, D] (each token's weight row contiguous), widened
    exactly; the product is a float64 matrix product (a library routine as
    one step of the definition)."""
    return _widen_bf16(hidden_bits) @ _widen_bf16(weight_bits).T


def lmhead_error_bound(hidden_bits, weight_bits) -> np.ndarray:
    """Bound on |z32 - z| for any binary32 evaluation that sums the D products
    h_d w_vd in any order: each product of two bf16 values is exact in
    binary32 (8-bit significands), and a sum of n terms in binary32, in any
    order and with or without fused multiply-adds, lies within
    gamma_{n-1} * sum |terms| of the exact sum, gamma_m = m u / (1 - m u),
    u = 2^-24 (Higham, "Accuracy and Stability of Numerical Algorithms",
    section 4.2)."""
    h = np.abs(_widen_bf16(hidden_bits))
    w = np.abs(_widen_bf16(weight_bits))
    D = h.shape[1]
    m = max(D - 1, 0)
    u = 2.0 ** -24
    return (m * u / (1.0 - m * u)) * (h @ w.T)


def lmhead_sample(hidden_bits, weight_bits, req, seed: int = 0, offset: int = 0, threads: int = 1,
                  exact: bool = False, rows=None):
    """The sampler applied to the LM head's logits: oracle.sample on the
    float64 logits rounded to binary32, plus `fragile` [B] bool: rows whose
    candidate list, kept count or token could change when every logit moves
    by up to its rounding bound (lmhead_error_bound + half an ulp of the
    value).  `exact`: inputs whose products and partial sums are all exact
    in binary32 (the bound is then zero and no row is fragile).  `rows`: only
    these rows are computed (the others' results are meaningless); each row
    keeps its own index in the noise counters."""
    h = np.asarray(hidden_bits)
    B = h.shape[0]
    V = np.asarray(weight_bits).shape[0]
    rows = list(range(B)) if rows is None else list(rows)
    zr = lmhead_logits(h[rows], weight_bits)
    z32 = np.zeros((B, V), np.float32)
    z32[rows] = zr.astype(np.float32)
    req = _lmhead_requests(req)
    out = sample(z32, 0, req, seed=seed, offset=offset, threads=threads)
    fragile = np.zeros(B, bool)
    if not exact:
        eps = lmhead_error_bound(h[rows], weight_bits) + np.abs(zr) * 2.0 ** -24
        for i, b in enumerate(rows):
            fragile[b] = _lmhead_row_fragile(zr[i], eps[i], out, b, req, seed, offset)
    out["fragile"] = fragile
    return out


def _lmhead_requests(req):
    """The LM-head step takes no side lists: a request asking for a grammar
    mask, or naming prior or bias entries, is an invalid row (expressed here
    as a stochastic row with a NaN temperature, which the sampler rejects)."""
    import copy
    r = copy.deepcopy(req)
    bad = r.use_grammar | (r.use_penalties & (r.n_prior > 0)) | (r.use_bias & (r.n_bias > 0))
    r.greedy = np.where(bad, False, r.greedy)
    r.temperature = np.where(bad, np.float32(np.nan), r.temperature).astype(np.float32)
    r.use_grammar = np.zeros_like(r.use_grammar)
    r.use_penalties = np.zeros_like(r.use_penalties)
    r.use_bias = np.zeros_like(r.use_bias)
    r.bitmask = None
    return r


def _lmhead_row_fragile(z, eps, out, b, req, seed, offset) -> bool:
    """Whether row b's token, kept count or set of candidates could change
    when every logit moves by up to `eps`: the boundary of the candidate set
    (rank K against rank K + 1; greedy rows: rank 1 against rank 2), then,
    for stochastic rows, the top-p and min-p cut decisions and the ranks on
    either side of the final cut, and the Gumbel-max margin, with v = z / T
    moving by at most max(eps) / T (float64 estimates with a small slack for
    the binary32 epilogue).  The order inside the candidate list is not
    checked: it changes neither the kept set's sums beyond the slack nor the
    token."""
    V = z.shape[0]
    if out["status"][b] not in (STATUS_OK, STATUS_TOPK_CLAMPED):
        return False
    K = int(min(req.top_k[b] if req.top_k[b] > 0 else KMAX, KMAX, V))
    order = np.lexsort((np.arange(V), -z))[:min(K + 1, V)]
    zs, es = z[order], eps[order]

    def split(r):   # ranks r and r + 1 (0-based) within the moves?
        return r + 1 < len(order) and zs[r] - zs[r + 1] <= es[r] + es[r + 1]

    greedy = bool(req.greedy[b]) or req.temperature[b] <= 0 or (req.top_k[b] == 1)
    if greedy:
        return split(0)
    if split(K - 1):
        return True
    T = float(req.temperature[b])
    dv = float(es[:K].max()) / T
    slack = 1e-6
    v = zs[:K] / T
    e = np.exp(v - v[0])
    Z = e.sum()
    E = np.concatenate([[0.0], np.cumsum(e)])
    n = K
    if req.top_p[b] < 1.0:
        p = float(req.top_p[b])
        n_p = int(np.sum(E[:K] < p * Z))
        for k in (n_p, n_p + 1):   # the last kept and the first dropped rank
            if 1 <= k <= K and abs(E[k - 1] - p * Z) <= (4 * dv + slack) * Z:
                return True
        n = min(n, n_p)
    if req.min_p[b] > 0.0:
        L = np.log(float(req.min_p[b]))
        n_m = int(np.sum(v - v[0] >= L))
        for k in (n_m, n_m + 1):
            if 1 <= k <= K and abs(v[k - 1] - v[0] - L) <= 2 * dv + slack:
                return True
        n = min(n, n_m)
    if n < K and split(n - 1):
        return True
    ids = order[:n]
    g = np.array([float(gumbel(seed, offset, int(i), b, 0)) for i in ids])
    s = v[:n] + g
    if n >= 2:
        s2 = np.sort(s)
        if s2[-1] - s2[-2] <= 2 * dv + slack * max(1.0, abs(s2[-1])):
            return True
    return False
