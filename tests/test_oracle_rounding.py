"""Pins of the oracle's rounding to narrow formats against independent
library conversions (numpy fp32 cast, Python's IEEE half packing, torch's CPU
bfloat16 cast)."""
import struct

import numpy as np
import torch

import oracle as O


def _random_f32(n, seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    return x[np.isfinite(x)]


def test_p24_matches_numpy_float32_cast():
    rng = np.random.default_rng(3)
    y = rng.standard_normal(200_000) * np.exp(rng.uniform(-105, 85, 200_000))
    # include exact float32 halfway points (ties) in both parities
    f = rng.standard_normal(20_000).astype(np.float32).astype(np.float64)
    ulp = np.spacing(f.astype(np.float32)).astype(np.float64)
    ties = np.concatenate([f + ulp / 2, f - ulp / 2])
    for v in (y, ties):
        assert np.array_equal(O.round_to_format(v, 24, -126),
                              v.astype(np.float32).astype(np.float64))


def test_f16_matches_python_half_packing():
    x = _random_f32(60_000, 4)
    x = np.concatenate([x, np.float32([65504, 65519.99, 65520, -65520, 2 ** -24,
                                       2 ** -25, 3 * 2 ** -26, 2 ** -26, 0.0, -0.0])])
    # exact fp16 midpoints
    h = np.arange(0, 0x7BFF, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
    hn = np.nextafter(h.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    x = np.concatenate([x, ((h + hn) / 2).astype(np.float32)])
    got = O.f32_to_f16_value(x)

    def ref(v):
        v = float(v)
        if abs(v) >= 65520.0:
            return np.copysign(np.inf, v)
        return struct.unpack("<e", struct.pack("<e", v))[0]
    want = np.array([ref(v) for v in x])
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_bf16_matches_torch_cast():
    x = _random_f32(1 << 21, 5)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(O.f32_to_bf16_value(x), want)


def test_bf16_ties_go_to_even():
    # 1 + 2**-8 is halfway between 1 and 1 + 2**-7: even mantissa is 1.0
    assert O.f32_to_bf16_value(np.float32(1 + 2 ** -8)) == 1.0
    # 1 + 3 * 2**-8 is halfway between 1 + 2**-7 (odd) and 1 + 2**-6 (even)
    assert O.f32_to_bf16_value(np.float32(1 + 3 * 2 ** -8)) == 1 + 2 ** -6


def test_bits_helpers_round_trip():
    v = O.f32_to_bf16_value(_random_f32(10_000, 6))
    v = v[np.isfinite(v)]
    assert np.array_equal(O.bf16_bits_to_f64(O.bf16_bits(v)), v)
    h = O.f32_to_f16_value(_random_f32(10_000, 7))
    h = h[np.isfinite(h)]
    assert np.array_equal(O.f16_bits(h).view(np.float16).astype(np.float64), h)
