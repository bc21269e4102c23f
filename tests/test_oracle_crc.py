"""Pins of the oracle's CRC-32: the catalogue check value, zlib, the
bit-at-a-time form, and tamper detection per record."""
import zlib

import numpy as np

import oracle as O


def test_check_value():
    assert O.crc32_bitwise(b"123456789") == 0xCBF43926
    rec = np.frombuffer(b"123456789", dtype=np.uint8)[None]
    assert int(O.crc32_records(rec)[0]) == 0xCBF43926


def test_matches_zlib_and_bitwise():
    rng = np.random.default_rng(41)
    for n in (1, 2, 3, 15, 16, 17, 255, 1000, 4096):
        recs = rng.integers(0, 256, (5, n)).astype(np.uint8)
        got = O.crc32_records(recs)
        for i in range(5):
            assert int(got[i]) == zlib.crc32(recs[i].tobytes())
        assert O.crc32_bitwise(recs[0].tobytes()) == int(got[0])
    big = rng.integers(0, 256, (3, 33280)).astype(np.uint8)
    got = O.crc32_records(big)
    assert [int(c) for c in got] == [zlib.crc32(r.tobytes()) for r in big]


def test_tamper_changes_only_that_record():
    rng = np.random.default_rng(42)
    recs = rng.integers(0, 256, (2, 6, 2048)).astype(np.uint8)
    base = O.crc32_records(recs)
    for trial in range(20):
        t = recs.copy()
        l, b, j, bit = rng.integers(2), rng.integers(6), rng.integers(2048), rng.integers(8)
        t[l, b, j] ^= np.uint8(1 << bit)
        c = O.crc32_records(t)
        diff = np.argwhere(c != base)
        assert diff.tolist() == [[l, b]]
    # a burst of up to 32 bits inside one record is always detected
    t = recs.copy()
    t[1, 3, 100:104] ^= np.uint8(0xFF)
    assert O.crc32_records(t)[1, 3] != base[1, 3]
