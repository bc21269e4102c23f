"""Pins of the oracle's RoPE and relative shift: the HyperCache post's float32
shift-error figure, the SO(2) identity and its consequences (identity at
zero, composition, norm), RoPE's relative-position property, the sign
convention and the split-halves convention as a permutation."""
import numpy as np

import oracle as O
from conftest import load_golden
from quantization_rope_reuse_amd import workloads as W

IL, HS = O.PAIRS_INTERLEAVED, O.PAIRS_HALF_SPLIT


def test_float32_shift_error_reproduces_printed_figure():
    """Keys of 64 tokens x 8 heads from a seed-0 generator, RoPE at 1024 + t,
    shifted by 7168, against RoPE at 8192 + t, all in float32 arithmetic with
    float64 angles: the max error prints as the post's 4.77e-07."""
    g = load_golden("hypercache_part_b.json")
    k, _ = W.tiny_pre_rope_kv()
    pos = W.tiny_positions()
    old = O.rope_apply(k, pos, 10000.0, IL)
    assert old.dtype == np.float32
    shifted = O.rope_shift(old, 7168, 10000.0, IL)
    direct = O.rope_apply(k, pos + 7168, 10000.0, IL)
    err = float(np.max(np.abs(shifted - direct)))
    assert float(f"{err:.{g['rope_shift_error_printed_digits'] - 1}e}") == \
        g["rope_shift_error_pos_1024_to_8192_float32"]
    assert float(f"{err:.1e}") >= g["rope_shift_error_text_approx"]
    # the float64 oracle itself is far tighter
    k64 = k.astype(np.float64)
    e64 = np.max(np.abs(O.rope_shift(O.rope_apply(k64, pos, 1e4, IL), 7168, 1e4, IL)
                        - O.rope_apply(k64, pos + 7168, 1e4, IL)))
    assert e64 < 1e-10


def test_zero_shift_is_identity_bit_for_bit():
    x = np.random.default_rng(31).standard_normal((16, 8, 128))
    for pairs in (IL, HS):
        assert np.array_equal(O.rope_shift(x, 0, 5e5, pairs), x)


def test_composition_and_norm():
    rng = np.random.default_rng(32)
    x = rng.standard_normal((32, 8, 128))
    for pairs in (IL, HS):
        for d1, d2 in ((512, -512), (16384, -3), (-4096, 4095), (7168, 1)):
            two = O.rope_shift(O.rope_shift(x, d1, 1e6, pairs), d2, 1e6, pairs)
            one = O.rope_shift(x, d1 + d2, 1e6, pairs)
            assert np.max(np.abs(two - one)) < 1e-11
        y = O.rope_shift(x, 12345, 1e4, pairs)
        ia, ib = O.pair_indices(pairs)
        n0 = x[..., ia] ** 2 + x[..., ib] ** 2
        n1 = y[..., ia] ** 2 + y[..., ib] ** 2
        assert np.max(np.abs(n0 - n1)) < 1e-12 * np.max(n0) * 10


def test_shift_equals_strip_then_apply():
    rng = np.random.default_rng(33)
    x = rng.standard_normal((64, 8, 128))
    m_old = 64 * 3 + np.arange(64)
    for pairs, base in ((IL, 1e4), (HS, 5e5)):
        post = O.rope_apply(x, m_old, base, pairs)
        back = O.rope_strip(post, m_old, base, pairs)
        assert np.max(np.abs(back - x)) < 1e-12
        via = O.rope_apply(O.rope_strip(post, m_old, base, pairs), m_old + 8192, base, pairs)
        direct = O.rope_shift(post, 8192, base, pairs)
        assert np.max(np.abs(via - direct)) < 1e-11


def test_relative_position_property_of_scores():
    """<R_m q, R_n k> depends only on m - n: the property RoPE is built for."""
    rng = np.random.default_rng(34)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    for pairs in (IL, HS):
        s0 = np.sum(O.rope_apply(q, [100], 1e4, pairs) * O.rope_apply(k, [37], 1e4, pairs))
        s1 = np.sum(O.rope_apply(q, [100 + 5000], 1e4, pairs) * O.rope_apply(k, [37 + 5000], 1e4, pairs))
        s2 = np.sum(O.rope_apply(q, [100 + 1], 1e4, pairs) * O.rope_apply(k, [37], 1e4, pairs))
        assert abs(s0 - s1) < 1e-10
        assert abs(s0 - s2) > 1e-6


def test_theta_and_sign_convention():
    for base in (1e4, 5e5, 1e6):
        th = O.rope_theta(base)
        assert th[0] == 1.0 and th.shape == (64,)
        r = th[1:] / th[:-1]
        assert np.allclose(r, base ** (-2 / 128), rtol=1e-13, atol=0)
        assert abs(th[-1] * base ** (126 / 128) - 1) < 1e-13
    # a quarter turn maps (a, b) to (-b, a): pair 0 has theta 1, so position
    # pi/2 is not an integer; use the rotation directly.
    x = np.zeros((1, 128))
    x[0, 0], x[0, 1] = 3.0, 5.0
    ang = np.zeros((1, 64))
    ang[0, 0] = np.pi / 2
    y = O.rotate_pairs(x, ang, IL)
    assert abs(y[0, 0] + 5.0) < 1e-15 and abs(y[0, 1] - 3.0) < 1e-15


def test_half_split_is_interleaved_on_permuted_vector():
    rng = np.random.default_rng(35)
    x = rng.standard_normal((8, 4, 128))
    perm = np.empty(128, dtype=np.int64)        # interleaved slot -> half-split slot
    perm[0::2] = np.arange(64)
    perm[1::2] = np.arange(64) + 64
    a = O.rope_shift(x, -1234, 1e6, HS)
    b = O.rope_shift(x[..., perm], -1234, 1e6, IL)
    assert np.array_equal(a[..., perm], b)
