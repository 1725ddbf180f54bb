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
