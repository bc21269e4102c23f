"""Pins of the oracle's recompute selection: the per-token drift norm against
integer Pythagorean rows and math.hypot, and the top-k selection against a
brute-force search over subsets and worked cases."""
import itertools
import math

import numpy as np
import pytest

import oracle as O


def test_drift_pythagorean_rows():
    cached = np.zeros((4, 6))
    fresh = np.zeros((4, 6))
    fresh[0, :2] = (3, 4)                       # 5
    fresh[1, :3] = (1, 2, 2)                    # 3
    fresh[2, :3] = (2, 3, 6)                    # 7
    fresh[3, :4] = (1, 4, 8, 0)                 # 9
    cached[3] = 10.0                            # shift both rows: still 9
    fresh[3] += 10.0
    assert O.token_drift(cached, fresh).tolist() == [5.0, 3.0, 7.0, 9.0]


def test_drift_against_hypot():
    rng = np.random.default_rng(61)
    a = rng.standard_normal((16, 37))
    b = a + rng.standard_normal((16, 37)) * rng.uniform(0.01, 2.0, (16, 1))
    got = O.token_drift(a, b)
    for t in range(16):
        want = math.hypot(*[float(y) - float(x) for x, y in zip(a[t], b[t])])
        assert abs(got[t] - want) <= 4e-16 * want


def test_drift_invariants():
    rng = np.random.default_rng(62)
    a = rng.standard_normal((8, 64))
    b = rng.standard_normal((8, 64))
    c = rng.standard_normal((8, 64))
    assert np.array_equal(O.token_drift(a, b), O.token_drift(b, a))
    assert not O.token_drift(a, a).any()
    assert np.array_equal(O.token_drift(4 * a, 4 * b), 4 * O.token_drift(a, b))
    assert (O.token_drift(a, c) <= O.token_drift(a, b) + O.token_drift(b, c) + 1e-12).all()


def test_drift_narrow_formats_convert_exactly():
    rng = np.random.default_rng(63)
    a = rng.standard_normal((3, 32)).astype(np.float16)
    b = (a.astype(np.float32) + 0.25).astype(np.float16)
    want = [math.hypot(*[float(y) - float(x) for x, y in zip(a[t], b[t])]) for t in range(3)]
    got = O.token_drift(a, b)
    assert np.allclose(got, want, rtol=4e-16, atol=0)


def test_recompute_count():
    assert [O.recompute_count(n) for n in (0, 1, 6, 7, 20, 100, 1280)] == [0, 0, 0, 1, 3, 15, 192]
    for n in range(1, 5000, 37):
        assert abs(O.recompute_count(n) - 0.15 * n) < 1.0


def _outranks(v, i, j):
    """Independent comparator: does token i come before token j?"""
    if math.isnan(v[i]) != math.isnan(v[j]):
        return math.isnan(v[i])
    if not math.isnan(v[i]) and v[i] != v[j]:
        return v[i] > v[j]
    return i < j


def _brute_force(v, k):
    winners = []
    for subset in itertools.combinations(range(len(v)), k):
        rest = [j for j in range(len(v)) if j not in subset]
        if all(_outranks(v, i, j) for i in subset for j in rest):
            winners.append(list(subset))
    assert len(winners) == 1
    return winners[0]


@pytest.mark.parametrize("seed", range(6))
def test_selection_brute_force(seed):
    rng = np.random.default_rng(70 + seed)
    n = int(rng.integers(1, 9))
    # few distinct values so that ties are common; some NaN and signed zeros
    pool = np.array([0.0, -0.0, 1.5, 1.5, 2.0, -3.0, np.nan, 7.0])
    v = [float(x) for x in rng.choice(pool, size=n)]
    for k in range(n + 1):
        got = O.select_top_tokens(v, k).tolist()
        assert got == _brute_force(v, k), (v, k)


def test_selection_worked_cases():
    assert O.select_top_tokens([2.0] * 6, 4).tolist() == [0, 1, 2, 3]
    assert O.select_top_tokens([1.0, 2.0], 0).tolist() == []
    assert O.select_top_tokens([5.0, 1.0, 3.0], 3).tolist() == [0, 1, 2]
    assert O.select_top_tokens([1.0, np.nan, np.inf, 0.5], 2).tolist() == [1, 2]
    assert O.select_top_tokens([-0.0, 0.0, -0.0], 2).tolist() == [0, 1]
    assert O.select_top_tokens([-1.0, -5.0, -0.5, -2.0], 2).tolist() == [0, 2]
    assert O.select_top_tokens([0.1, 0.9, 0.4, 0.9, 0.2], 3).tolist() == [1, 2, 3]
    sel = O.select_top_tokens(np.arange(100.0)[::-1], 15)
    assert sel.dtype == np.int32 and sel.tolist() == list(range(15))
    with pytest.raises(ValueError):
        O.select_top_tokens([1.0, 2.0], 3)
