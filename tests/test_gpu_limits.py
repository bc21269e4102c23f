"""GPU parity at the ABI's size limits.

* One block of 2^24 vectors, the most a block may hold (2^20 tokens x 16
  heads), through the put and the fetch.  Its FP8 record is 4.36 GB, and its
  V codes start 2^31 bytes in.  Sampled vectors (the first, the last, around
  the K/V boundary, and random ones) go through the oracle.  Every page
  vector must be written and finite.  The CRC calls refuse a record this large.
* The largest record the CRC calls accept: 258,048 tokens x 16 heads, FP8,
  1,073,479,680 bytes.  It runs through the CRC kernel and the fused put +
  CRC, compared with zlib's CRC-32 of the record and with the plain put's
  bytes."""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import oracle as O
from parity_util import (check_keys, check_values_exact, crc_u32, canary_fill, host_f64,
                         is_canary)
from quantization_rope_reuse_amd import hkv

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _source(tb, H, seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    k = torch.randn((1, 1, tb, H, 128), dtype=torch.bfloat16, device=DEV, generator=gen)
    v = torch.randn((1, 1, tb, H, 128), dtype=torch.bfloat16, device=DEV, generator=gen)
    return k, v


def _sample_vectors(vecs, rng, n=64):
    picks = {0, 1, vecs // 2 - 1, vecs // 2, vecs - 2, vecs - 1}
    picks.update(int(x) for x in rng.integers(0, vecs, size=n))
    return np.array(sorted(picks), dtype=np.int64)


def _check_sampled(rec, k, v, ko, vo, fmt, H, vs_idx, dm, base, pairs):
    """Oracle on the sampled vectors of block 0 (page 0 for the put and the
    fetch): codes and scale bytes in the record, fetched V exact, K in
    tolerance."""
    vecs = k.shape[2] * H
    cb = 128 if fmt == "fp8" else 64
    flat = rec.view(-1)
    idx = torch.from_numpy(vs_idx).to(DEV)
    for kv, src, out in ((0, k, ko), (1, v, vo)):
        x = host_f64(src.view(-1, 128)[idx]).astype(np.float32)            # [n, 128]
        quant = O.quant_fp8_vectors if fmt == "fp8" else O.quant_int4_vectors
        codes, scale = quant(x)
        cbase = kv * vecs * cb
        cidx = (cbase + idx[:, None] * cb + torch.arange(cb, device=DEV)[None]).reshape(-1)
        got_codes = flat[cidx].view(len(vs_idx), cb).cpu().numpy()
        assert np.array_equal(got_codes, codes.reshape(len(vs_idx), cb)), f"kv {kv}: codes differ"
        sbase = 2 * vecs * cb + 2 * kv * vecs
        sidx = (sbase + 2 * idx[:, None] + torch.arange(2, device=DEV)[None]).reshape(-1)
        got_s = flat[sidx].view(len(vs_idx), 2).cpu().numpy().view("<u2").reshape(-1)
        assert np.array_equal(got_s, O.f16_bits(scale).astype(np.uint16).reshape(-1)), \
            f"kv {kv}: scales differ"
        deq = (O.e4m3_value(codes) if fmt == "fp8" else
               O.int4_unpack(codes).astype(np.float64)) * np.asarray(scale)[..., None]
        got = host_f64(out.view(-1, 128)[idx])
        if kv == 1:
            check_values_exact(got, O.round_output(deq, "bf16"), "V")
        else:
            exact = O.rope_shift(deq, float(dm), base, pairs)
            check_keys(got, exact, deq, "bf16", "K")


@pytest.mark.parametrize("fmt", ["fp8", "int4"])
def test_block_of_2_24_vectors(fmt):
    tb, H = 1 << 20, 16
    print(f"[limits] 2^24-vector block {fmt}", flush=True)
    k, v = _source(tb, H, 101)
    table = torch.zeros(1, dtype=torch.int32, device=DEV)
    rec = hkv.alloc_records(1, 1, fmt, tb, H, device=DEV)
    assert rec.shape[-1] == hkv.record_bytes(fmt, tb, H) > (1 << 31)
    (hkv.quant_fp8 if fmt == "fp8" else hkv.quant_int4)(k, v, table, rec)
    dm_val = 123457
    dm = torch.full((1,), dm_val, dtype=torch.int32, device=DEV)
    ko = canary_fill(torch.empty_like(k))
    vo = canary_fill(torch.empty_like(v))
    hkv.fetch_dequant_rope_shift(rec, fmt, table, dm, 500000.0, "half_split", ko, vo)
    torch.cuda.synchronize()
    _check_sampled(rec, k, v, ko, vo, fmt, H, _sample_vectors(tb * H, np.random.default_rng(7)),
                   dm_val, 500000.0, "half_split")
    for out in (ko, vo):
        assert not bool(is_canary(out).any()), "a page vector was not written"
        assert bool(torch.isfinite(out).all()), "non-finite output"
    with pytest.raises(hkv.HkvError) as e:
        hkv.crc32_blocks(rec, fmt, tb, H)
    assert e.value.status == hkv.ERR_UNSUPPORTED
    del k, v, rec, ko, vo
    torch.cuda.empty_cache()


def test_largest_crc_record():
    tb, H = 258048, 16
    rb = hkv.record_bytes("fp8", tb, H)
    assert rb == 1073479680 <= (1 << 30) < hkv.record_bytes("fp8", tb + 1024, H)
    print("[limits] largest CRC record", flush=True)
    k, v = _source(tb, H, 103)
    table = torch.zeros(1, dtype=torch.int32, device=DEV)
    rec = hkv.alloc_records(1, 1, "fp8", tb, H, device=DEV)
    fused = hkv.alloc_records(1, 1, "fp8", tb, H, device=DEV)
    hkv.quant_fp8(k, v, table, rec)
    crc = hkv.crc32_blocks(rec, "fp8", tb, H)
    crc_fused = hkv.quant_crc("fp8", k, v, table, fused)
    torch.cuda.synchronize()
    assert torch.equal(rec, fused), "the fused put wrote different bytes"
    want = zlib.crc32(rec.cpu().numpy().tobytes())
    assert int(crc_u32(crc)[0, 0]) == want, "CRC kernel differs from zlib"
    assert int(crc_u32(crc_fused)[0, 0]) == want, "fused CRC differs from zlib"
    ko = canary_fill(torch.empty_like(k))
    vo = canary_fill(torch.empty_like(v))
    dm = torch.full((1,), -77777, dtype=torch.int32, device=DEV)
    hkv.fetch_dequant_rope_shift(rec, "fp8", table, dm, 10000.0, "interleaved", ko, vo)
    torch.cuda.synchronize()
    _check_sampled(rec, k, v, ko, vo, "fp8", H, _sample_vectors(tb * H, np.random.default_rng(11)),
                   -77777, 10000.0, "interleaved")
    del k, v, rec, fused, ko, vo
    torch.cuda.empty_cache()
