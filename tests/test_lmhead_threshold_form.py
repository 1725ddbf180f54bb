"""The thresholded LM-head GEMM keeps a value v of row r when its merge key
ord32(canon(v)) exceeds the row's threshold key; the kernel tests this as a
float compare, v > t, with t the key's canonical value (FLT_MAX raised to
+inf, the no-candidate key 0xFFFFFFFF read as a NaN).  This checks that the
two forms agree on every class of binary32 pattern (zeros of both signs,
subnormals, normals, FLT_MAX, infinities, NaNs of both signs) against every
threshold a full probe tile can give (the key of any canonical value, -inf
to FLT_MAX) and the no-candidate key.
"""
import numpy as np

F32_MAX = 0x7F7FFFFF
PINF, NINF = 0x7F800000, 0xFF800000


def canon_bits(u):
    u = u.astype(np.uint32)
    f = u.view(np.float32)
    out = u.copy()
    out[np.isnan(f)] = NINF
    out[u == PINF] = F32_MAX
    out[u == 0x80000000] = 0
    return out


def ord32(u):
    u = u.astype(np.uint32)
    return np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)


def unord32(k):
    k = k.astype(np.uint32)
    return np.where(k & 0x80000000, k & 0x7FFFFFFF, ~k).astype(np.uint32)


def test_float_compare_matches_key_compare():
    rng = np.random.default_rng(5)
    special = np.array([0, 0x80000000, 1, 0x80000001, 0x007FFFFF, 0x807FFFFF, 0x00800000, 0x80800000,
                        0x3F800000, 0xBF800000, F32_MAX, F32_MAX | 0x80000000, PINF, NINF,
                        0x7FC00000, 0xFFC00000, 0x7F800001, 0xFF800001, 0x7FFFFFFF, 0xFFFFFFFF], np.uint32)
    vals = np.concatenate([special, rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)])
    # thresholds: keys of canonical values (from the same patterns), and the no-candidate key
    th_src = canon_bits(np.concatenate([special, rng.integers(0, 2**32, 300, dtype=np.uint64).astype(np.uint32)]))
    keys = np.unique(np.concatenate([ord32(th_src), np.array([0xFFFFFFFF], np.uint32)]))
    vkey = ord32(canon_bits(vals))
    vf = vals.view(np.float32)
    for k in keys:
        t = unord32(np.array([k], np.uint32))
        if t[0] == F32_MAX:
            t = np.array([PINF], np.uint32)
        tf = t.view(np.float32)[0]
        with np.errstate(invalid="ignore"):
            by_float = vf > tf
        by_key = vkey > k
        assert np.array_equal(by_float, by_key), hex(int(k))
