"""The fp32-reciprocal division the kernels use to split a vector index into
(token, head): q = trunc(fl(fl(v) * fl(1/d))), r = v - q*d, then one
correction each way.  Checked here with the same IEEE fp32 operations in
numpy against integer division, over every v in [0, 2^24 + 64] for small
divisors and a spread of large ones (head counts are at most 2^24 / 1)."""
import numpy as np


def _divmod_small(v, d):
    rcp = np.float32(1.0) / np.float32(d)
    q = (v.astype(np.float32) * rcp).astype(np.int64)       # fp32 product, truncated
    r = v - q * d
    neg = r < 0
    q[neg] -= 1
    r[neg] += d
    big = r >= d
    q[big] += 1
    r[big] -= d
    return q, r


def test_divmod_small_matches_integer_division():
    v_all = np.arange((1 << 24) + 65, dtype=np.int64)
    divisors = list(range(1, 41)) + [63, 64, 65, 96, 127, 255, 257, 1000, 4099, 65535, 65537,
                                     (1 << 20) + 7, (1 << 23) - 1, (1 << 23) + 1, (1 << 24) - 3,
                                     1 << 24]
    for d in divisors:
        for lo in range(0, v_all.size, 1 << 22):
            v = v_all[lo:lo + (1 << 22)]
            q, r = _divmod_small(v, d)
            assert np.array_equal(q, v // d), f"quotient, d={d}"
            assert np.array_equal(r, v % d), f"remainder, d={d}"
