"""ctypes binding of libss (include/ss.h).

Argument marshalling only: every step of the sampling path runs in the HIP
kernels of libss.so.  Functions take torch tensors that already live on the
GPU (PyTorch provides device memory and streams) and pass their data
pointers to the C ABI.  If the library is not built, importing this module
raises - there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libss.so")

SS_F32 = 0
SS_BF16 = 1
KMAX = 128
GAMMA_MAX = 16

SS_OK = 0
SS_ERR_INVALID_ARG = -1
SS_ERR_UNSUPPORTED = -2
SS_ERR_WORKSPACE = -3
SS_ERR_HIP = -4
SS_ERR_NOALLOC_LIMIT = -5
NOALLOC_WS_BYTES = 16 << 20

ROW_OK = 0
ROW_ALL_MASKED = 1
ROW_INVALID = 2
ROW_TOPK_CLAMPED = 3

SS_GREEDY = 1 << 0
SS_GRAMMAR = 1 << 1
SS_REP = 1 << 2
SS_FREQPRES = 1 << 3
SS_BIAS = 1 << 4
SS_TOPK = 1 << 5
SS_TOPP = 1 << 6
SS_MINP = 1 << 7

# struct ss_req (32 bytes)
SS_REQ = np.dtype([
    ("flags", "<u2"), ("top_k", "<u2"), ("temperature", "<f4"), ("n_prior", "<u2"), ("n_bias", "<u2"),
    ("top_p", "<f4"), ("min_p", "<f4"), ("rep_penalty", "<f4"), ("freq_penalty", "<f4"),
    ("pres_penalty", "<f4"),
])
assert SS_REQ.itemsize == 32


class SsAux(ctypes.Structure):
    _fields_ = [
        ("prior_ids", ctypes.c_void_p), ("prior_cnt", ctypes.c_void_p), ("prior_stride", ctypes.c_int32),
        ("bias_ids", ctypes.c_void_p), ("bias_val", ctypes.c_void_p), ("bias_stride", ctypes.c_int32),
        ("bitmask", ctypes.c_void_p), ("bitmask_stride", ctypes.c_int64),
    ]


class LibraryMissing(RuntimeError):
    pass


def _load():
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                             "python -m speculative_decoding_verification_stage1_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, u64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t
    L.ss_workspace_bytes.argtypes = [i32, i32, i32]
    L.ss_workspace_bytes.restype = sz
    L.ss_tile_size.argtypes = [i32]
    L.ss_tile_size.restype = i32
    L.ss_sample_step.argtypes = [P, i32, i32, i32, i64, P, P, P, u64, P, P, P, P, P, P, P, sz, P]
    L.ss_sample_step.restype = i32
    L.ss_sample_step_noalloc.argtypes = [P, i32, i32, i32, i64, P, P, P, u64, P, P, P, P, P, P, P]
    L.ss_sample_step_noalloc.restype = i32
    L.ss_verify_step.argtypes = [P, i32, i32, i32, i32, i64, P, P, P, u64, P, P, P, P, P, P, sz, P]
    L.ss_verify_step.restype = i32
    L.ss_verify_step_var.argtypes = [P, i32, i32, i32, i32, i64, P, P, P, u64, P, P, P, P, P, P, P, sz, P]
    L.ss_verify_step_var.restype = i32
    L.ss_verify_dense_workspace_bytes.argtypes = [i32, i32, i32]
    L.ss_verify_dense_workspace_bytes.restype = sz
    L.ss_verify_step_dense.argtypes = [P, i32, i32, i32, i32, i64, P, P, u64, P, P, P, P, P, P, P, sz, P]
    L.ss_verify_step_dense.restype = i32
    L.ss_stream_read.argtypes = [P, sz, i32, P, P]
    L.ss_stream_read.restype = i32
    L.ss_topk_step.argtypes = [P, i32, i32, i32, i64, i32, P, P, P, sz, P]
    L.ss_topk_step.restype = i32
    L.ss_topk_step_radix.argtypes = [P, i32, i32, i32, i64, i32, P, P, P, sz, P]
    L.ss_topk_step_radix.restype = i32
    L.ss_topk_single_pass.argtypes = [P, i32, i32, i32, i64, i32, P, P, P]
    L.ss_topk_single_pass.restype = i32
    L.ss_tile_topk.argtypes = [P, i32, i32, i32, i64, i32, P, P, P, P, sz, P]
    L.ss_tile_topk.restype = i32
    L.ss_rng_advance.argtypes = [P, u64, P]
    L.ss_rng_advance.restype = i32
    L.ss_lmhead_workspace_bytes.argtypes = [i32, i32]
    L.ss_lmhead_workspace_bytes.restype = sz
    L.ss_lmhead_logits.argtypes = [P, i64, P, i64, i32, i32, i32, P, i64, P]
    L.ss_lmhead_logits.restype = i32
    L.ss_lmhead_sample_step.argtypes = [P, i64, P, i64, i32, i32, i32, P, P, u64, P, P, P, P, P, P, P, sz, P]
    L.ss_lmhead_sample_step.restype = i32
    L.ss_spec_eval.argtypes = [i32, ctypes.c_uint32, i64, ctypes.c_uint32, ctypes.c_uint32, u64, u64, P, P]
    L.ss_spec_eval.restype = i32
    L.ss_status_str.argtypes = [i32]
    L.ss_status_str.restype = ctypes.c_char_p
    return L


lib = _load()

EXPORTS = ["ss_workspace_bytes", "ss_tile_size", "ss_sample_step", "ss_sample_step_noalloc", "ss_verify_step", "ss_verify_step_var",
           "ss_verify_dense_workspace_bytes", "ss_verify_step_dense", "ss_topk_step", "ss_topk_step_radix",
           "ss_topk_single_pass", "ss_tile_topk", "ss_lmhead_workspace_bytes", "ss_lmhead_logits",
           "ss_lmhead_sample_step", "ss_spec_eval", "ss_rng_advance", "ss_stream_read", "ss_status_str"]


class SsError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"libss error {code}: {lib.ss_status_str(code).decode()}")
        self.code = code


def _check(rc: int) -> int:
    if rc != SS_OK:
        raise SsError(rc)
    return rc


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def ptr(t) -> int | None:
    """Device (or host) address of a torch tensor, None for None."""
    return None if t is None else t.data_ptr()


def stream_handle(stream=None) -> int | None:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def flags_of(req, i: int) -> int:
    f = 0
    if req.greedy[i]:
        f |= SS_GREEDY
    if req.use_grammar[i]:
        f |= SS_GRAMMAR
    if req.use_penalties[i]:
        f |= SS_REP | SS_FREQPRES
    if req.use_bias[i]:
        f |= SS_BIAS
    if req.top_k[i] > 0:
        f |= SS_TOPK
    if req.top_p[i] < 1.0:
        f |= SS_TOPP
    if req.min_p[i] > 0.0:
        f |= SS_MINP
    return f


def pack_requests(req, flags=None) -> np.ndarray:
    """numpy array of struct ss_req from a workloads.Requests."""
    B = req.batch
    a = np.zeros(B, SS_REQ)
    a["flags"] = [flags_of(req, i) for i in range(B)] if flags is None else flags
    a["temperature"] = req.temperature
    a["top_k"] = np.clip(req.top_k, 0, 65535)
    a["n_prior"] = np.clip(req.n_prior, 0, 65535)
    a["n_bias"] = np.clip(req.n_bias, 0, 65535)
    a["top_p"] = req.top_p
    a["min_p"] = req.min_p
    a["rep_penalty"] = req.rep_penalty
    a["freq_penalty"] = req.freq_penalty
    a["pres_penalty"] = req.pres_penalty
    return a


class DeviceRequests:
    """Requests and their side arrays copied to the GPU."""

    def __init__(self, req, device="cuda", flags=None):
        import torch
        self.req_np = pack_requests(req, flags)
        self.req = torch.from_numpy(self.req_np.view(np.uint8).copy()).to(device)
        self.prior_ids = torch.from_numpy(np.ascontiguousarray(req.prior_ids, np.int32)).to(device)
        self.prior_cnt = torch.from_numpy(np.ascontiguousarray(req.prior_cnt, np.int32)).to(device)
        self.bias_ids = torch.from_numpy(np.ascontiguousarray(req.bias_ids, np.int32)).to(device)
        self.bias_val = torch.from_numpy(np.ascontiguousarray(req.bias_val, np.float32)).to(device)
        self.bitmask = None
        if req.bitmask is not None:
            self.bitmask = torch.from_numpy(np.ascontiguousarray(req.bitmask).view(np.int32)).to(device)
        self.aux = SsAux(ptr(self.prior_ids), ptr(self.prior_cnt), self.prior_ids.shape[1],
                         ptr(self.bias_ids), ptr(self.bias_val), self.bias_ids.shape[1],
                         ptr(self.bitmask), 0 if self.bitmask is None else self.bitmask.shape[1])

    def with_bitmask(self, bitmask_t):
        """Use another device bitmask tensor (int32 view of uint32 words)."""
        self.bitmask = bitmask_t
        self.aux.bitmask = ptr(bitmask_t)
        self.aux.bitmask_stride = bitmask_t.shape[1]
        return self


def make_rng(seed: int = 0, offset: int = 0, device="cuda"):
    import torch
    a = np.array([seed, offset], np.uint64).view(np.int64)
    return torch.from_numpy(a.copy()).to(device)


def workspace(rows: int, V: int, dtype: int, device="cuda", fill: int | None = None):
    """A workspace for `rows` rows of width V (torch allocations are
    256-byte aligned; the library needs no initialisation).  `fill` sets
    every byte, for tests that the library reads nothing it did not write."""
    import torch
    n = int(lib.ss_workspace_bytes(rows, V, dtype))
    t = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    if fill is not None:
        t.fill_(fill)
    return t


def dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SS_BF16
    if t.dtype == torch.float32:
        return SS_F32
    raise TypeError(f"unsupported logits dtype {t.dtype}")


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def ss_sample_step(logits, dreq: DeviceRequests, rng, out_tokens, out_topk_ids=None, out_probs=None,
                   out_kept=None, out_mass=None, out_status=None, ws=None, stream=None,
                   rng_advance: int = 0) -> int:
    B, V = logits.shape
    rc = lib.ss_sample_step(ptr(logits), dtype_code(logits), B, V, logits.stride(0), ptr(dreq.req),
                            ctypes.byref(dreq.aux), ptr(rng), rng_advance, ptr(out_tokens), ptr(out_topk_ids),
                            ptr(out_probs), ptr(out_kept), ptr(out_mass), ptr(out_status), ptr(ws),
                            0 if ws is None else ws.numel(), stream_handle(stream))
    return _check(rc)


def ss_sample_step_noalloc(logits, dreq: DeviceRequests, rng, out_tokens, out_topk_ids=None, out_probs=None,
                           out_kept=None, out_mass=None, out_status=None, stream=None,
                           rng_advance: int = 0) -> int:
    B, V = logits.shape
    rc = lib.ss_sample_step_noalloc(ptr(logits), dtype_code(logits), B, V, logits.stride(0), ptr(dreq.req),
                                    ctypes.byref(dreq.aux), ptr(rng), rng_advance, ptr(out_tokens),
                                    ptr(out_topk_ids), ptr(out_probs), ptr(out_kept), ptr(out_mass),
                                    ptr(out_status), stream_handle(stream))
    return _check(rc)


def ss_verify_step(target, B: int, gamma: int, dreq: DeviceRequests, rng, draft_ids, draft_probs,
                   out_tokens, out_n_emit, out_status=None, ws=None, stream=None,
                   rng_advance: int = 0) -> int:
    rows, V = target.shape
    rc = lib.ss_verify_step(ptr(target), dtype_code(target), B, gamma, V, target.stride(0), ptr(dreq.req),
                            ctypes.byref(dreq.aux), ptr(rng), rng_advance, ptr(draft_ids), ptr(draft_probs),
                            ptr(out_tokens), ptr(out_n_emit), ptr(out_status), ptr(ws),
                            0 if ws is None else ws.numel(), stream_handle(stream))
    return _check(rc)


def ss_verify_step_var(target, B: int, gamma: int, dreq: DeviceRequests, rng, cu_num_draft, draft_ids,
                       draft_probs, out_tokens, out_n_emit, out_status=None, ws=None, stream=None,
                       rng_advance: int = 0) -> int:
    rows, V = target.shape
    rc = lib.ss_verify_step_var(ptr(target), dtype_code(target), B, gamma, V, target.stride(0), ptr(dreq.req),
                                ctypes.byref(dreq.aux), ptr(rng), rng_advance, ptr(cu_num_draft), ptr(draft_ids),
                                ptr(draft_probs), ptr(out_tokens), ptr(out_n_emit), ptr(out_status), ptr(ws),
                                0 if ws is None else ws.numel(), stream_handle(stream))
    return _check(rc)


def dense_workspace(B: int, gamma: int, V: int, device="cuda", fill: int | None = None):
    """Workspace of ss_verify_step_dense (256-byte aligned torch allocation,
    no initialisation needed; `fill` as for workspace())."""
    import torch
    n = int(lib.ss_verify_dense_workspace_bytes(B, gamma, V))
    t = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    if fill is not None:
        t.fill_(fill)
    return t


def ss_verify_step_dense(target, B: int, gamma: int, dreq: DeviceRequests, rng, draft_ids, draft_probs,
                         out_tokens, out_n_emit, out_status=None, ws=None, cu_num_draft=None, stream=None,
                         rng_advance: int = 0) -> int:
    rows, V = target.shape
    rc = lib.ss_verify_step_dense(ptr(target), dtype_code(target), B, gamma, V, target.stride(0), ptr(dreq.req),
                                  ptr(rng), rng_advance, ptr(cu_num_draft), ptr(draft_ids), ptr(draft_probs),
                                  ptr(out_tokens), ptr(out_n_emit), ptr(out_status), ptr(ws),
                                  0 if ws is None else ws.numel(), stream_handle(stream))
    return _check(rc)


def ss_stream_read(buf, out, stream=None) -> int:
    """Streaming read of the whole tensor `buf` (the bandwidth reference);
    out: int32/uint32 tensor with one word per workgroup."""
    rc = lib.ss_stream_read(ptr(buf), buf.numel() * buf.element_size(), out.numel(), ptr(out), stream_handle(stream))
    return _check(rc)


def ss_topk_step(logits, k: int, out_ids, out_vals=None, ws=None, stream=None) -> int:
    B, V = logits.shape
    rc = lib.ss_topk_step(ptr(logits), dtype_code(logits), B, V, logits.stride(0), k, ptr(out_ids),
                          ptr(out_vals), ptr(ws), 0 if ws is None else ws.numel(), stream_handle(stream))
    return _check(rc)


def ss_topk_step_radix(logits, k: int, out_ids, out_vals=None, ws=None, stream=None) -> int:
    B, V = logits.shape
    rc = lib.ss_topk_step_radix(ptr(logits), dtype_code(logits), B, V, logits.stride(0), k, ptr(out_ids),
                                ptr(out_vals), ptr(ws), 0 if ws is None else ws.numel(), stream_handle(stream))
    return _check(rc)


def ss_topk_single_pass(logits, k: int, out_ids, out_vals=None, stream=None) -> int:
    B, V = logits.shape
    rc = lib.ss_topk_single_pass(ptr(logits), dtype_code(logits), B, V, logits.stride(0), k, ptr(out_ids),
                                 ptr(out_vals), stream_handle(stream))
    return _check(rc)


def ss_tile_topk(logits, rows_per_req: int = 1, dreq: DeviceRequests | None = None, out_ids=None,
                 ws=None, stream=None) -> int:
    rows, V = logits.shape
    rc = lib.ss_tile_topk(ptr(logits), dtype_code(logits), rows, V, logits.stride(0), rows_per_req,
                          None if dreq is None else ptr(dreq.req),
                          None if dreq is None else ctypes.byref(dreq.aux),
                          ptr(out_ids), ptr(ws), 0 if ws is None else ws.numel(), stream_handle(stream))
    return _check(rc)


def lmhead_workspace(B: int, V: int, device="cuda", fill: int | None = None):
    """Workspace of ss_lmhead_sample_step (no initialisation needed; `fill`
    as for workspace())."""
    import torch
    n = int(lib.ss_lmhead_workspace_bytes(B, V))
    t = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    if fill is not None:
        t.fill_(fill)
    return t


def _bf16_2d(t):
    import torch
    if t.dtype not in (torch.bfloat16, torch.int16):
        raise TypeError(f"LM-head operands are bf16 (or their int16 patterns), got {t.dtype}")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("LM-head operands are row-major 2-D tensors")
    return t


def ss_lmhead_logits(hidden, weight, out, stream=None) -> int:
    """out[b, v] = hidden[b] . weight[v] (fp32), hidden [B, D], weight [V, D]."""
    _bf16_2d(hidden)
    _bf16_2d(weight)
    B, D = hidden.shape
    V = weight.shape[0]
    rc = lib.ss_lmhead_logits(ptr(hidden), hidden.stride(0), ptr(weight), weight.stride(0), B, D, V, ptr(out),
                              out.stride(0), stream_handle(stream))
    return _check(rc)


def ss_lmhead_sample_step(hidden, weight, dreq: DeviceRequests, rng, out_tokens, out_topk_ids=None,
                          out_probs=None, out_kept=None, out_mass=None, out_status=None, ws=None, stream=None,
                          rng_advance: int = 0, D: int | None = None) -> int:
    _bf16_2d(hidden)
    _bf16_2d(weight)
    B = hidden.shape[0]
    D = hidden.shape[1] if D is None else D
    V = weight.shape[0]
    rc = lib.ss_lmhead_sample_step(ptr(hidden), hidden.stride(0), ptr(weight), weight.stride(0), B, D, V,
                                   ptr(dreq.req), ptr(rng), rng_advance, ptr(out_tokens), ptr(out_topk_ids),
                                   ptr(out_probs), ptr(out_kept), ptr(out_mass), ptr(out_status), ptr(ws),
                                   0 if ws is None else ws.numel(), stream_handle(stream))
    return _check(rc)


SS_SPEC_EXP, SS_SPEC_LOG, SS_SPEC_LOG_NORMAL, SS_SPEC_GUMBEL_WORD, SS_SPEC_PHILOX, SS_SPEC_GUMBEL = range(6)


def ss_spec_eval(fn: int, first: int, out, c1: int = 0, c2: int = 0, seed: int = 0, offset: int = 0,
                 stream=None) -> int:
    """out[i] = the device function fn at argument first + i (out: int32 or
    uint32 device tensor of n elements)."""
    rc = lib.ss_spec_eval(fn, first & 0xFFFFFFFF, out.numel(), c1, c2, seed, offset, ptr(out), stream_handle(stream))
    return _check(rc)


def ss_rng_advance(rng, delta: int, stream=None) -> int:
    return _check(lib.ss_rng_advance(ptr(rng), delta, stream_handle(stream)))


def ss_tile_size(dtype: int) -> int:
    return int(lib.ss_tile_size(dtype))


def ss_workspace_bytes(rows: int, V: int, dtype: int) -> int:
    return int(lib.ss_workspace_bytes(rows, V, dtype))
