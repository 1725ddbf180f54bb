"""Penalty histories and bias lists longer than 256 entries (GPU).

Requests may name up to SS_PRIOR_MAX = 4096 prior entries and
SS_BIAS_MAX = 1024 bias entries.  Lists of more than 256 entries are left
out of the tiles through the mask and ranked by their own launch; shorter
lists in the same call keep the Stage-1 path.  Each row below takes one
case (both lists at their limits with duplicates and ignored entries, just
past 256, short lists beside long strides, one past each limit, a grammar,
greedy, every listed id in one tile, negative logits); the per-tile lists
and the whole sampling step are checked against the oracle bit for bit, in
bf16 and fp32.  Verification with the drafts in a long penalty history is
checked the same way, with fixed and per-request draft counts.
"""
import numpy as np
import pytest
import torch

import oracle
from speculative_decoding_verification_stage1_amd import workloads as W

pytestmark = pytest.mark.gpu

PS, BS = 4100, 1030   # list strides (longer than the limits, to test them)


def _lib():
    from speculative_decoding_verification_stage1_amd import _lib
    return _lib


def _long_requests(n, V, rng):
    req = W.plain_requests(n, temperature=0.9, top_p=0.95, prior_len=PS, bias_len=BS)
    req.temperature[:] = rng.uniform(0.6, 1.4, n).astype(np.float32)
    req.use_penalties[:] = True
    req.rep_penalty[:] = 1.15
    req.freq_penalty[:] = 0.05
    req.pres_penalty[:] = 0.1
    req.use_bias[:] = True
    req.prior_ids = rng.integers(0, V, (n, PS)).astype(np.int32)   # duplicates happen
    req.prior_cnt = rng.integers(1, 6, (n, PS)).astype(np.int32)
    req.bias_ids = rng.integers(0, V, (n, BS)).astype(np.int32)
    req.bias_val = rng.uniform(-3, 3, (n, BS)).astype(np.float32)
    req.n_prior = np.full(n, 1000, np.int32)
    req.n_bias = np.full(n, 300, np.int32)
    # ignored entries: count 0, negative and out-of-range ids
    req.prior_cnt[:, 5::97] = 0
    req.prior_ids[:, 7::89] = -3
    req.prior_ids[:, 11::83] = V + 5
    req.bias_ids[:, 13::79] = -1
    return req


def _rows(V, rng):
    n = 12
    x = (rng.standard_normal((n, V)) * 2).astype(np.float32)
    req = _long_requests(n, V, rng)
    req.n_prior[0], req.n_bias[0] = 4096, 1024          # both at their limits
    req.n_prior[1], req.n_bias[1] = 300, 0              # just past 256
    req.use_bias[1] = False
    req.n_prior[2], req.n_bias[2] = 100, 200            # short lists, long strides
    req.n_prior[3] = 4097                               # past the limit: invalid
    req.n_bias[4] = 1025                                # past the limit: invalid
    bm = np.full((n, (V + 31) // 32), 0xFFFFFFFF, np.uint32)
    allowed = rng.random(V) < 0.3
    p = np.zeros(bm.shape[1] * 32, bool)
    p[:V] = allowed
    bm[5] = np.packbits(p, bitorder="little").view("<u4")
    req.use_grammar[5] = True                           # grammar + long lists
    req.bitmask = bm
    req.greedy[6] = True                                # greedy
    req.prior_ids[7, :4096] = np.arange(4096)           # every listed id in tile 0
    req.n_prior[7] = 4096
    x[7, :4096] += 3.0
    z = x[8].astype(np.float64)                         # log-softmax row
    x[8] = (z - (z.max() + np.log(np.exp(z - z.max()).sum()))).astype(np.float32)
    req.prior_ids[9, :2000] = req.prior_ids[9, 0]       # one id repeated 2000 times
    req.n_prior[9] = 2000
    req.top_k[10] = 40
    req.min_p[11] = 0.05
    return x, req


def _dev(x, dtype):
    return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16) if dtype == W.DTYPE_BF16 \
        else torch.from_numpy(x).cuda()


@pytest.mark.parametrize("dtype", [W.DTYPE_BF16, W.DTYPE_F32])
def test_long_lists_sample(dtype):
    from test_gpu_parity import same_bits
    lib = _lib()
    rng = np.random.default_rng(77)
    V = 70001
    x, req = _rows(V, rng)
    logits = W.to_bf16_bits(x) if dtype == W.DTYPE_BF16 else x
    xd = _dev(logits, dtype)
    dreq = lib.DeviceRequests(req)
    # tile view (the step's first launch)
    tile = lib.ss_tile_size(dtype)
    Zv = (V + tile - 1) // tile
    out = torch.full((12, Zv, 128), -7, dtype=torch.int32, device="cuda")
    lib.ss_tile_topk(xd, 1, dreq, out, lib.workspace(12, V, dtype, fill=0x5C))
    torch.cuda.synchronize()
    ref = oracle.tile_topk(logits, dtype, tile, req)
    bad = np.argwhere((out.cpu().numpy() != ref).any(axis=2))
    assert len(bad) == 0, bad[:10].tolist()
    # the step
    o = dict(tokens=torch.full((12,), -7, dtype=torch.int32, device="cuda"),
             topk_ids=torch.full((12, 128), -7, dtype=torch.int32, device="cuda"),
             probs=torch.full((12, 128), -7.0, dtype=torch.float32, device="cuda"),
             kept=torch.full((12,), -7, dtype=torch.int32, device="cuda"),
             mass=torch.full((12,), -7.0, dtype=torch.float32, device="cuda"),
             status=torch.full((12,), -7, dtype=torch.int32, device="cuda"))
    lib.ss_sample_step(xd, dreq, lib.make_rng(3, 1), o["tokens"], o["topk_ids"], o["probs"], o["kept"], o["mass"],
                       o["status"], lib.workspace(12, V, dtype, fill=0xA7))
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in o.items()}
    r = oracle.sample(logits, dtype, req, seed=3, offset=1, threads=16)
    assert list(r["status"][3:5]) == [oracle.STATUS_INVALID] * 2
    for i in range(12):
        for k in ("status", "topk_ids", "kept", "tokens"):
            assert np.array_equal(g[k][i], r[k][i]), (k, i)
        same_bits(g["probs"][i], r["probs"][i], str(i))
        same_bits(g["mass"][i], r["mass"][i], str(i))


def test_long_history_verify():
    from test_gpu_parity import verify_parity, _counts_cu
    V = 30000
    wl = W.workload_verify(B=8, gamma=4, V=V)
    rng = np.random.default_rng(78)
    req = _long_requests(8, V, rng)
    req.greedy[:] = False
    req.greedy[::3] = True
    req.temperature[:] = 1.0
    req.top_p[:] = 1.0
    req.n_prior = np.array([4096, 3000, 257, 100, 4096, 2048, 600, 0], np.int32)
    req.n_bias = np.array([1024, 0, 0, 50, 512, 300, 1024, 700], np.int32)
    # drafts that hit prior entries, and repeated drafts
    req.prior_ids[1::2, :2] = wl.draft_ids[1::2, :2]
    wl.draft_ids[2, 3] = wl.draft_ids[2, 1]
    req.prior_cnt[3, 0] = 0
    req.prior_ids[3, 0] = wl.draft_ids[3, 0]            # a draft meeting an ignored entry
    wl.req = req
    flags = [oracle.flags_of(req, b) | (oracle.FLAG_DRAFT_HIST if b % 2 == 0 else 0) for b in range(8)]
    verify_parity(wl, seed=6, offset=2, flags=flags)
    verify_parity(wl, seed=6, offset=2, flags=flags, cu_num_draft=_counts_cu(rng.integers(0, 5, 8)))
