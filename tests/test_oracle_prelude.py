"""Pins of the oracle's logits-processing prelude (CPU only).

The SonicSampler paper (section 3.1 "Logits processing") names the steps -
grammar mask, repetition penalty, frequency/presence penalties, logit bias -
but not their formulas; the readings used are the CTRL repetition rule and
additive penalties.  Pins: a hand-worked example with exact binary32 values
(``tests/golden/prelude_worked_example.txt``), special cases that reduce to
the identity, canonicalisation of special values, bf16 widening against
torch's bfloat16 conversion, and monotonicity in the penalty parameters.
"""
import os

import numpy as np
import torch

import oracle
from speculative_decoding_verification_stage1_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    vals = {}
    with open(os.path.join(GOLDEN, "prelude_worked_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, *v = line.split()
            vals[k] = v
    return vals


def _req_one(V, prior, bias, rep=2.0, freq=0.25, pres=0.5):
    r = W.plain_requests(1, prior_len=max(1, len(prior)), bias_len=max(1, len(bias)))
    for j, (i, c) in enumerate(prior):
        r.prior_ids[0, j] = i
        r.prior_cnt[0, j] = c
    r.n_prior[0] = len(prior)
    for j, (i, b) in enumerate(bias):
        r.bias_ids[0, j] = i
        r.bias_val[0, j] = b
    r.n_bias[0] = len(bias)
    r.rep_penalty[:] = rep
    r.freq_penalty[:] = freq
    r.pres_penalty[:] = pres
    return r


def test_worked_example():
    g = _golden()
    x = np.array([float(v) for v in g["x"]], np.float32)
    r = _req_one(8, [(0, 2), (1, 1), (5, 0), (3, 3)], [(3, 1.0), (6, -4.0)])
    flags = oracle.FLAG_REP | oracle.FLAG_FREQPRES | oracle.FLAG_BIAS
    z = oracle.prelude_row(x, W.DTYPE_F32, flags, r, 0)
    assert np.array_equal(z, np.array([float(v) for v in g["z"]], np.float32))
    out = oracle.sample(x[None], W.DTYPE_F32, r, flags=[flags | oracle.FLAG_GREEDY])
    order = [int(v) for v in g["order"]]
    assert list(out["topk_ids"][0, :8]) == order
    assert out["tokens"][0] == order[0]
    # grammar mask allowing ids {0,1,2,5,6}
    bm = np.array([[0x67]], np.uint32)
    zm = oracle.prelude_row(x, W.DTYPE_F32, flags | oracle.FLAG_GRAMMAR, r, 0, bitmask_row=bm[0])
    assert np.array_equal(zm, np.array([float(v) for v in g["masked_z"]], np.float32))
    r.bitmask = bm
    out = oracle.sample(x[None], W.DTYPE_F32, r, flags=[flags | oracle.FLAG_GRAMMAR | oracle.FLAG_GREEDY])
    assert list(out["topk_ids"][0, :8]) == [int(v) for v in g["masked_order"]]


def test_identity_special_cases():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(4096).astype(np.float32) * 3
    prior = [(int(i), int(c)) for i, c in zip(rng.choice(4096, 64, replace=False), rng.integers(1, 6, 64))]
    bias = [(int(i), 0.0) for i in rng.choice(4096, 16, replace=False)]
    r = _req_one(4096, prior, bias, rep=1.0, freq=0.0, pres=0.0)
    allf = oracle.FLAG_REP | oracle.FLAG_FREQPRES | oracle.FLAG_BIAS | oracle.FLAG_GRAMMAR
    bm = np.full(128, 0xFFFFFFFF, np.uint32)
    z = oracle.prelude_row(x, W.DTYPE_F32, allf, r, 0, bitmask_row=bm)
    assert np.array_equal(z, x)
    # all-zero mask -> everything -inf
    z0 = oracle.prelude_row(x, W.DTYPE_F32, oracle.FLAG_GRAMMAR, r, 0, bitmask_row=np.zeros(128, np.uint32))
    assert np.all(z0 == -np.inf)
    # masked tokens stay -inf through every penalty and bias
    r2 = _req_one(4096, prior, [(i, 5.0) for i, _ in bias], rep=1.3, freq=0.2, pres=0.1)
    z1 = oracle.prelude_row(x, W.DTYPE_F32, allf, r2, 0, bitmask_row=np.zeros(128, np.uint32))
    assert np.all(z1 == -np.inf)


def test_canonical_special_values():
    x = np.array([np.nan, np.inf, -0.0, -np.inf, 1.5, -np.nan], np.float32)
    r = W.plain_requests(1)
    z = oracle.prelude_row(x, W.DTYPE_F32, 0, r, 0)
    assert z[0] == -np.inf and z[3] == -np.inf and z[5] == -np.inf
    assert z[1] == np.finfo(np.float32).max
    assert z[2] == 0.0 and not np.signbit(z[2])
    assert z[4] == 1.5


def test_bf16_widening_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, 50000, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    z = oracle.prelude_row(bits, W.DTYPE_BF16, 0, W.plain_requests(1), 0)
    fin = np.isfinite(ref)
    expect = ref.copy()
    expect[np.isnan(ref)] = -np.inf
    expect[ref == np.inf] = np.finfo(np.float32).max
    expect[ref == 0] = 0.0
    assert np.array_equal(z, expect)
    assert fin.sum() > 40000


def test_penalty_monotonicity():
    """Larger theta, counts or presence can only lower a listed logit;
    a positive bias raises it; unlisted tokens never change."""
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(512) * 4).astype(np.float32)
    ids = rng.choice(512, 32, replace=False)
    base = None
    for theta in [1.0, 1.1, 1.5, 3.0]:
        r = _req_one(512, [(int(i), 2) for i in ids], [], rep=theta, freq=0.0, pres=0.0)
        z = oracle.prelude_row(x, W.DTYPE_F32, oracle.FLAG_REP, r, 0)
        if base is not None:
            assert np.all(z[ids] <= base[ids])
        mask = np.ones(512, bool)
        mask[ids] = False
        assert np.array_equal(z[mask], x[mask])
        base = z
    zc = []
    for c in [1, 2, 3, 4, 5]:
        r = _req_one(512, [(int(i), c) for i in ids], [], rep=1.0, freq=0.2, pres=0.1)
        zc.append(oracle.prelude_row(x, W.DTYPE_F32, oracle.FLAG_FREQPRES, r, 0)[ids])
    for a, b in zip(zc, zc[1:]):
        assert np.all(b < a)
        np.testing.assert_allclose(a - b, 0.2, rtol=0, atol=1e-5)
    r = _req_one(512, [], [(int(i), 2.5) for i in ids], rep=1.0)
    zb = oracle.prelude_row(x, W.DTYPE_F32, oracle.FLAG_BIAS, r, 0)
    np.testing.assert_allclose(zb[ids] - x[ids], 2.5, atol=1e-5)


def test_workload_generator_shapes():
    wl = W.workload_mixed(2, 4, 4096, grammar=True)
    assert wl.logits.dtype == np.uint16 and wl.logits.shape == (4, 4096)
    assert wl.req.bitmask.shape == (4, 128)
    frac = np.unpackbits(wl.req.bitmask.view(np.uint8), bitorder="little").mean()
    assert 0.03 < frac < 0.08
    # one of the raw top-10 is allowed in every row
    raw = W.bf16_bits_to_f32(wl.logits)
    for r in range(4):
        top = np.argsort(-raw[r], kind="stable")[:16]
        bits = (wl.req.bitmask[r][top >> 5] >> (top & 31)) & 1
        assert bits.any()
    assert wl.req.greedy.sum() == 2
