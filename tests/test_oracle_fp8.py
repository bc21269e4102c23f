"""Pins of the oracle's E4M3FN decoder and encoder: the format definition's
landmarks, torch's CPU float8_e4m3fn conversion, every rounding midpoint and
the exact round trip of representable values.  Two exhaustive sweeps close
the loop through the threshold fixture, which equals the closed-form midpoint
rule: torch's conversion of every finite fp32 value (clamped to +-448), and
the oracle's encoder on every fp32 pattern from 0 to 448."""
import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import torch

import oracle as O
from conftest import load_golden
from fp8_sweep import expected_steps, observed_steps, oracle_chunk_ok

BITS_448 = 0x43E00000          # fp32 pattern of 448.0, the largest finite E4M3FN value
BITS_INF = 0x7F800000          # first non-finite positive pattern


def _torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy())
    return t.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def _torch_encode(x):
    x = np.clip(np.asarray(x, dtype=np.float32), -448, 448)
    return torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_table_matches_torch():
    codes = np.arange(256)
    ours = O.e4m3_value(codes)
    ref = _torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_format_landmarks():
    v = O.e4m3_value(np.array([0x7E, 0x08, 0x07, 0x01, 0x00, 0x80, 0x38, 0xFE]))
    assert v[0] == 448.0 and v[1] == 2.0 ** -6 and v[2] == 7 * 2.0 ** -9
    assert v[3] == 2.0 ** -9 and v[4] == 0.0 and np.signbit(v[5]) and v[5] == 0.0
    assert v[6] == 1.0 and v[7] == -448.0


def test_round_trip_of_every_representable_value():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    vals = O.e4m3_value(codes).astype(np.float32)
    assert np.array_equal(O.e4m3_encode(vals), codes.astype(np.uint8))


def test_encoder_matches_torch_on_random_patterns():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # bias half the sample into the format's range so that rounding is exercised
    y = (rng.standard_normal(1 << 21) * np.exp(rng.uniform(-12, 7, 1 << 21))).astype(np.float32)
    for v in (x, y):
        assert np.array_equal(O.e4m3_encode(v), _torch_encode(v))


def test_every_midpoint_rounds_to_even_mantissa():
    codes = np.arange(0, 126)
    lo = O.e4m3_value(codes)
    hi = O.e4m3_value(codes + 1)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)   # exact in fp32
    want = np.where(codes % 2 == 0, codes, codes + 1).astype(np.uint8)
    assert np.array_equal(O.e4m3_encode(mid), want)
    below = np.nextafter(mid, np.float32(0))
    above = np.nextafter(mid, np.float32(np.inf))
    assert np.array_equal(O.e4m3_encode(below), codes.astype(np.uint8))
    assert np.array_equal(O.e4m3_encode(above), (codes + 1).astype(np.uint8))
    assert np.array_equal(O.e4m3_encode(-mid), want | 0x80)
    for v in (mid, below, above):
        assert np.array_equal(O.e4m3_encode(v), _torch_encode(v))


def test_saturation_and_signed_zero():
    big = np.float32([448.0, 448.01, 463.99, 464.0, 465.0, 1e30, 3.4e38, np.inf])
    assert np.all(O.e4m3_encode(big) == 0x7E)
    assert np.all(O.e4m3_encode(-big) == 0xFE)
    tiny = np.float32([0.0, 1e-30, 2.0 ** -10, 1e-45])
    assert np.all(O.e4m3_encode(tiny) == 0x00)
    assert np.all(O.e4m3_encode(-tiny) == 0x80)


def test_threshold_fixture_matches_midpoint_rule():
    """The stored thresholds (written from the oracle) equal the closed-form
    rule: the first pattern above code c is the midpoint itself when the tie
    goes up (c odd) and the next pattern when it stays (c even)."""
    th = np.array(load_golden("fp8_thresholds.json")["first_bits_above_code"], dtype=np.int64)
    codes = np.arange(126)
    mid = ((O.e4m3_value(codes) + O.e4m3_value(codes + 1)) / 2).astype(np.float32)
    mid_bits = mid.view(np.uint32).astype(np.int64)
    assert np.array_equal(th, mid_bits + (codes % 2 == 0))


def test_encoder_monotone_in_positive_bit_pattern():
    rng = np.random.default_rng(12)
    bits = np.sort(rng.integers(0, 0x43E00001, size=1 << 20, dtype=np.int64))
    c = O.e4m3_encode(bits.astype(np.uint32).view(np.float32)).astype(np.int64)
    assert np.all(np.diff(c) >= 0)
    th = np.array(load_golden("fp8_thresholds.json")["first_bits_above_code"], dtype=np.int64)
    assert np.array_equal(c, np.searchsorted(th, bits, side="right"))


def test_torch_cast_matches_fixture_on_every_finite_value():
    """Every finite fp32 value, both signs: torch's float8_e4m3fn conversion of
    the value clamped to +-448 is the fixture's code of |x|, with the sign bit
    for negative x (including -0)."""
    th = np.array(load_golden("fp8_thresholds.json")["first_bits_above_code"], dtype=np.int64)
    chunk = 1 << 24
    for start in range(0, BITS_INF, chunk):
        end = min(start + chunk, BITS_INF)
        x = np.arange(start, end, dtype=np.int64).astype(np.uint32).view(np.float32)
        np.clip(x, 0.0, 448.0, out=x)
        pos = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got_first, got_steps = observed_steps(pos, start)
        want_first, want_steps = expected_steps(th, start, end)
        assert got_first == want_first and np.array_equal(got_steps, want_steps), \
            f"torch and the fixture differ in [{start:#x}, {end:#x})"
        np.negative(x, out=x)
        neg = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(neg, pos | 0x80), f"sign handling differs in [{start:#x}, {end:#x})"


def test_oracle_encoder_matches_fixture_on_every_pattern_up_to_448():
    """The oracle's encoder on all 1,138,753,537 fp32 patterns from +0 to 448
    against the fixture, in chunks over a pool of worker processes."""
    th = load_golden("fp8_thresholds.json")["first_bits_above_code"]
    chunk = 1 << 22
    jobs = [(s, min(s + chunk, BITS_448 + 1), th) for s in range(0, BITS_448 + 1, chunk)]
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    ctx = multiprocessing.get_context("spawn")
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        bad = [j[:2] for j, ok in zip(jobs, ex.map(oracle_chunk_ok, jobs)) if not ok]
    assert not bad, f"oracle and fixture differ in chunks {bad[:3]}"
