"""Pins of the oracle's frame container: the header bytes spelled out with
struct from the layout, the header and payload CRCs against zlib, and each
kind of damage raising its own verification flag."""
import struct
import zlib

import numpy as np
import pytest

import oracle as O


def _spelled(fmt_code, tb, heads, layer, block, m_old, nbytes, crc):
    body = struct.pack("<IHHBBHHHIIiII24x", 0x46564B48, 1, 64, fmt_code, 0, 128, tb, heads,
                       layer, block, m_old, nbytes, crc)
    assert len(body) == 60
    return body + struct.pack("<I", zlib.crc32(body))


def test_header_bytes_spelled_out():
    got = O.frame_header("fp8", 64, 8, 3, 17, -5, 133120, 0xDEADBEEF).tobytes()
    assert got == _spelled(0, 64, 8, 3, 17, -5, 133120, 0xDEADBEEF)
    got = O.frame_header("int4", 16, 2, 0, 65535, 1 << 30, 4224, 7).tobytes()
    assert got == _spelled(1, 16, 2, 0, 65535, 1 << 30, 4224, 7)
    assert got[:4] == b"HKVF"


def test_header_round_trip():
    h = O.frame_header("int4", 64, 8, 31, 255, -2**31, 67584, 0xFFFFFFFF)
    f = O.parse_frame_header(h)
    assert (f["format"], f["block_tokens"], f["n_kv_heads"], f["layer"], f["block"]) == \
        (1, 64, 8, 31, 255)
    assert f["m_old"] == -2**31 and f["payload_crc"] == 0xFFFFFFFF
    assert f["header_crc"] == zlib.crc32(h[:60].tobytes())


def _frames(fmt="fp8", L=2, nb=5, tb=4, H=2, seed=0):
    rng = np.random.default_rng(seed)
    rb = O.record_bytes(fmt, tb, H)
    rec = rng.integers(0, 256, (L, nb, rb)).astype(np.uint8)
    m_old = rng.integers(0, 1 << 20, nb).astype(np.int32)
    return rec, m_old, O.make_frames(rec, fmt, tb, H, m_old, layer_base=4)


def test_make_frames_layout():
    rec, m_old, fr = _frames()
    assert fr.shape == (2, 5, 64 + rec.shape[2])
    assert np.array_equal(fr[:, :, 64:], rec)
    for l in range(2):
        for b in range(5):
            h = O.parse_frame_header(fr[l, b, :64])
            assert h["payload_crc"] == zlib.crc32(rec[l, b].tobytes())
            assert (h["layer"], h["block"], h["m_old"]) == (4 + l, b, int(m_old[b]))
            assert h["payload_bytes"] == rec.shape[2]


def test_verify_flags_each_kind_of_damage():
    rec, m_old, fr = _frames("int4")
    ok = O.verify_frames(fr, "int4", 4, 2, layer_base=4)
    assert not ok.any()
    # magic
    t = fr.copy()
    t[0, 1, 0] ^= 1
    f = O.verify_frames(t, "int4", 4, 2, layer_base=4)
    assert f[0, 1] == O.FRAME_BAD_MAGIC | O.FRAME_BAD_HEADER_CRC and f.sum() == f[0, 1]
    # a consistent but wrong header (its CRC recomputed): geometry only
    t = fr.copy()
    t[1, 2, 12] = 8
    t[1, 2, 60:64] = np.frombuffer(struct.pack("<I", zlib.crc32(t[1, 2, :60].tobytes())),
                                   dtype=np.uint8)
    f = O.verify_frames(t, "int4", 4, 2, layer_base=4)
    assert f[1, 2] == O.FRAME_BAD_GEOMETRY and f.sum() == f[1, 2]
    # header CRC word itself
    t = fr.copy()
    t[0, 0, 62] ^= 0x80
    f = O.verify_frames(t, "int4", 4, 2, layer_base=4)
    assert f[0, 0] == O.FRAME_BAD_HEADER_CRC and f.sum() == f[0, 0]
    # one payload bit
    t = fr.copy()
    t[1, 4, 64 + 37] ^= 0x10
    f = O.verify_frames(t, "int4", 4, 2, layer_base=4)
    assert f[1, 4] == O.FRAME_BAD_PAYLOAD_CRC and f.sum() == f[1, 4]
    # two frames swapped: both intact, both in the wrong slot
    t = fr.copy()
    t[0, [1, 3]] = t[0, [3, 1]]
    f = O.verify_frames(t, "int4", 4, 2, layer_base=4)
    assert f[0, 1] == f[0, 3] == O.FRAME_BAD_INDEX and f.sum() == 2 * O.FRAME_BAD_INDEX
    # read as the wrong format / layer
    assert (O.verify_frames(fr, "fp8", 4, 2, layer_base=4) & O.FRAME_BAD_GEOMETRY).all()
    assert (O.verify_frames(fr, "int4", 4, 2, layer_base=0) == O.FRAME_BAD_INDEX).all()


@pytest.mark.parametrize("fmt", ["fp8", "int4"])
def test_frame_delta(fmt):
    rec, m_old, fr = _frames(fmt)
    m_new = m_old.astype(np.int64) + np.array([0, 7168, -512, 512, 1])
    assert O.frame_delta_m(fr, m_new).tolist() == [0, 7168, -512, 512, 1]
    # clamped to int32
    t = O.make_frames(rec[:, :2], fmt, 4, 2, np.array([-2**31, 2**31 - 1]))
    assert O.frame_delta_m(t, [2**31 - 1, -2**31]).tolist() == [2**31 - 1, -2**31]
