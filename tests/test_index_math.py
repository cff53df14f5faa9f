"""The write kernels divide a row index t = token * nkv + head by nkv with a
multiply and a shift instead of an integer-divide sequence: m = ceil(2^(32+s)
/ n) with 2^s >= n, t / n = (t * m) >> (32 + s), claimed exact for
0 <= t < 2^31 (the write paths reject more rows).  This checks that claim
for head counts 1..130 and a large one, on every t near a multiple of n up to
2^31 - 1 and on random t."""
import numpy as np


def _magic(n):
    s = 0
    while (1 << s) < n:
        s += 1
    return ((1 << (32 + s)) + n - 1) // n, 32 + s


def test_magic_division_exact():
    r = np.random.default_rng(7)
    top = (1 << 31) - 1
    for n in list(range(1, 131)) + [1000, 65535, 65536, 65537]:
        m, sh = _magic(n)
        assert m < (1 << 33)                      # t * m stays below 2^64
        q_top = top // n
        qs = np.unique(np.concatenate([np.arange(0, 2000), q_top - np.arange(0, 2000),
                                       r.integers(0, q_top + 1, 4000)]))
        ts = (qs[:, None] * n + np.array([0, n - 1])[None, :]).ravel()   # both ends of each quotient
        ts = np.concatenate([ts, r.integers(0, top + 1, 20000), [top]])
        ts = ts[(ts >= 0) & (ts <= top)].astype(object)
        got = np.array([(int(t) * m) >> sh for t in ts], dtype=object)
        want = np.array([int(t) // n for t in ts], dtype=object)
        assert np.array_equal(got, want), n
