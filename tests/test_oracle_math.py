"""Pins of the oracle's arithmetic building blocks (CPU only).

* Philox4x32-10 against the published known-answer vectors
  (``tests/golden/philox4x32_10_kat.txt``) and against rocRAND's own
  host-side Philox engine, compiled from the installed ROCm header at test
  time (an independent implementation of the same published generator).
* exp/log against float64 libm (numpy) over strided sweeps of every fp32
  bit pattern in the domain the sampler uses, plus dense windows around the
  edges; the bound is 2 ulp.
* The uniform mapping u = ((w >> 9) + 1/2) 2^-23: end points and exactness.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            assert parts[0] == "philox4x32" and parts[1] == "10"
            vals = [int(p, 16) for p in parts[2:]]
            rows.append((vals[0:4], vals[4:6], vals[6:10]))
    return rows


@pytest.mark.parametrize("ctr,key,expect", _kat())
def test_philox_known_answers(ctr, key, expect):
    assert list(oracle.philox(ctr, key)) == expect


ROCRAND_PROBE = r"""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
int main() {
  const unsigned long long seeds[] = {0ull, 1ull, 0x0123456789abcdefull, 0xffffffffffffffffull};
  const unsigned long long subseq[] = {0ull, 5ull, 0x00000007000000ffull};
  const unsigned long long offs[] = {0ull, 4ull * 9ull, 4ull * 0x100000003ull};
  for (auto s : seeds) for (auto q : subseq) for (auto o : offs) {
    rocrand_state_philox4x32_10 st;
    rocrand_init(s, q, o, &st);
    uint4 v = rocrand4(&st);
    std::printf("%llx %llx %llx %08x %08x %08x %08x\n", s, q, o, v.x, v.y, v.z, v.w);
  }
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_philox_matches_rocrand_host_engine():
    """rocRAND's engine draws block i of subsequence q with counter
    (i_lo, i_hi, q_lo, q_hi) and key (seed_lo, seed_hi); the oracle's Philox
    must give the same four words for every such counter/key."""
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "probe.cpp")
        exe = os.path.join(d, "probe")
        with open(src, "w") as f:
            f.write(ROCRAND_PROBE)
        subprocess.run(["hipcc", "-O1", "-o", exe, src], check=True, capture_output=True, timeout=600)
        out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=60).stdout
    n = 0
    for line in out.strip().splitlines():
        s, q, o, *w = line.split()
        s, q, o = int(s, 16), int(q, 16), int(o, 16)
        blk = o // 4
        ctr = [blk & 0xFFFFFFFF, blk >> 32, q & 0xFFFFFFFF, q >> 32]
        key = [s & 0xFFFFFFFF, s >> 32]
        assert list(oracle.philox(ctr, key)) == [int(x, 16) for x in w], line
        n += 1
    assert n == 36


def _ulp32(ref64):
    """Spacing of binary32 at |ref| (for normal results)."""
    r = np.abs(ref64).astype(np.float32)
    return np.spacing(r).astype(np.float64)


def _sweep(lo_bits, hi_bits, stride):
    bits = np.arange(lo_bits, hi_bits, stride, dtype=np.uint64).astype(np.uint32)
    return bits.view(np.float32)


SWEEP_CHUNK = 1 << 23


def _chunk_err(fn, a, n, ref_fn):
    x = np.arange(a, a + n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    y = oracle.spec_sweep(fn, a, n).view(np.float32).astype(np.float64)
    ref = ref_fn(x.astype(np.float64))
    nz = ref != 0
    err = np.zeros(n)
    err[nz] = np.abs(y[nz] - ref[nz]) / _ulp32(ref[nz])
    i = int(np.argmax(err))
    return float(err[i]), float(x[i])


def _max_ulp_err(fn, lo_bits, hi_bits, ref_fn):
    """Largest error in binary32 ulps of the oracle's fn over EVERY float
    with bits in [lo_bits, hi_bits), against ref_fn in float64 (chunks in
    a thread pool: the oracle's C and numpy's loops release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    starts = range(lo_bits, hi_bits, SWEEP_CHUNK)
    with ThreadPoolExecutor(max_workers=os.cpu_count() or 1) as ex:
        res = list(ex.map(lambda a: _chunk_err(fn, a, min(SWEEP_CHUNK, hi_bits - a), ref_fn), starts))
    return max(res)


def test_exp_spec_within_2ulp():
    # every float from -0 (0x80000000) down to -86 (0xC2AC0000): the
    # arguments x = v - v_1 the epilogue can pass above the cut
    worst, at = _max_ulp_err(oracle.SWEEP_EXP, 0x80000000, 0xC2AC0001, np.exp)
    assert worst <= 2.0, (worst, at)
    assert oracle.exp_spec(0.0) == 1.0
    assert oracle.exp_spec(-np.inf) == 0.0
    assert oracle.exp_spec(-86.5) == 0.0
    # below the cut: every float from -86 (exclusive) to -inf gives 0
    assert not np.any(oracle.spec_sweep(oracle.SWEEP_EXP, 0xC2AC0001, 0xFF800001 - 0xC2AC0001,
                                        threads=os.cpu_count() or 1))
    # monotone on a dense grid (a written polynomial can step back by an
    # ulp between neighbouring floats; the grid's steps are far wider)
    g = np.linspace(-20, 0, 400001, dtype=np.float32)
    assert np.all(np.diff(oracle.exp_spec_n(g).astype(np.float64)) >= 0)


def test_log_spec_within_2ulp():
    # every positive finite float, subnormals included
    worst, at = _max_ulp_err(oracle.SWEEP_LOG, 1, 0x7F800000, np.log)
    assert worst <= 2.0, (worst, at)
    g = np.linspace(1e-6, 20, 400001, dtype=np.float32)
    assert np.all(np.diff(oracle.log_spec_n(g).astype(np.float64)) >= 0)
    assert oracle.log_spec(1.0) == 0.0
    assert oracle.log_spec(0.0) == -np.inf
    assert oracle.log_spec(np.inf) == np.inf
    assert np.isnan(oracle.log_spec(-1.0))


def test_uniform_mapping():
    lo = oracle.uniform(0)
    hi = oracle.uniform(0xFFFFFFFF)
    assert lo == np.float32(2.0 ** -24)
    assert hi == np.float32(1.0 - 2.0 ** -24)
    # exactness: (k + 1/2) * 2^-23 for k = w >> 9
    for w in [1 << 9, 12345 << 9, (1 << 32) - 512, 0x80000000]:
        k = w >> 9
        assert float(oracle.uniform(w)) == (k + 0.5) * 2.0 ** -23


def test_gumbel_moments():
    """Standard Gumbel: mean = Euler-Mascheroni gamma, variance pi^2/6."""
    g = np.array([oracle.gumbel(7, 3, i, 11, 0) for i in range(60000)], np.float64)
    assert abs(g.mean() - 0.5772156649) < 0.02
    assert abs(g.var() - np.pi ** 2 / 6) < 0.05
