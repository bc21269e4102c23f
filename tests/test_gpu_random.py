"""Seeded random configurations through the whole path, against the oracle.

Each seed draws a configuration and runs put (plain or fused with the
CRC), the CRC kernel and a fetch, checking everything against the CPU
oracle.  A configuration fixes:
* format, source and page dtypes, pair convention and RoPE base;
* layers, blocks, tokens per block and heads (ragged and 64-aligned shapes);
* padded and head-major page strides, and padded record strides;
* put tables with skipped, out-of-range and repeated entries;
* fetch tables over a random subset of pages;
* visit order (none, by page, or random);
* per-block or per-token deltas, from small to the ends of the int32 range.

Bar, as in the other parity tests: records and CRCs bit-exact; values, and
keys of blocks with a zero delta, exact; other keys within 2e-6 * ||k||
(fp32 pages) or one unit in the last place (16-bit pages).  Untouched records
and pages keep their fill bytes."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from parity_util import (TORCH_OF, canary_fill, check_keys, check_values_exact,
                         compare_fetch_block, crc_u32, host_f64, is_canary)
from quantization_rope_reuse_amd import hkv

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SEEDS = range(48)


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def _pages(L, P, tb, H, dtype, rng):
    """Uninitialised pages [L, P, tb, H, 128] of `dtype` with padded strides,
    token-major or head-major (a transposed view)."""
    es = torch.finfo(dtype).bits // 8
    pad = int(rng.choice([0, 1, 2])) * (16 // es)        # keeps every stride 16-byte aligned
    extra = int(rng.integers(0, 2))                      # spare pages in the buffer
    if rng.random() < 0.5:
        base = torch.empty((L, P + extra, tb, H, 128 + pad), dtype=dtype, device=DEV)
        return base[:, :P, :, :, :128]
    base = torch.empty((L, P + extra, H, tb, 128 + pad), dtype=dtype, device=DEV)
    return base[:, :P, :, :, :128].transpose(2, 3)


def _draw(seed):
    rng = np.random.default_rng([131, seed])
    c = dict(
        fmt=str(rng.choice(["fp8", "int4"])),
        src=str(rng.choice(["f32", "f16", "bf16"])),
        dst=str(rng.choice(["f32", "f16", "bf16"])),
        pairs=str(rng.choice(["interleaved", "half_split"])),
        base=float(rng.choice([10000.0, 500000.0, 1e6, 123.5])),
        L=int(rng.integers(1, 4)),
        P=int(rng.integers(1, 9)),
        fused=bool(rng.random() < 0.6),
        order=str(rng.choice(["none", "page", "random"])),
        per_token=bool(rng.random() < 0.3),
        scale=float(10.0 ** rng.uniform(-3, 3)),
    )
    if c["src"] == "f16":                 # keep the x20 channels finite in fp16 (max 65504)
        c["scale"] = min(c["scale"], 300.0)
    if rng.random() < 0.5:                                # whole-chunk shapes: one-pass fusion
        c["tb"], c["H"] = [(8, 8), (16, 8), (64, 8), (32, 4), (16, 16)][int(rng.integers(0, 5))]
    else:
        c["tb"], c["H"] = int(rng.integers(1, 70)), int(rng.integers(1, 17))
    c["nb"] = int(rng.integers(1, c["P"] + 3))
    return c, rng


@pytest.mark.parametrize("seed", SEEDS)
def test_random_configuration(seed):
    c, rng = _draw(seed)
    print(f"[random] seed {seed}: {c}", flush=True)
    L, P, tb, H, nb, fmt = c["L"], c["P"], c["tb"], c["H"], c["nb"], c["fmt"]

    # sources: N(0, scale^2), a few channels x20
    kp = rng.standard_normal((L, P, tb, H, 128)) * c["scale"]
    vp = rng.standard_normal((L, P, tb, H, 128)) * c["scale"]
    hot = rng.integers(0, H * 128, size=2)
    kp.reshape(L, P, tb, H * 128)[..., hot] *= 20
    src_k = _pages(L, P, tb, H, TORCH_OF[c["src"]], rng)
    src_v = torch.empty_strided(src_k.shape, src_k.stride(), dtype=src_k.dtype, device=DEV)
    src_k.copy_(torch.from_numpy(kp.astype(np.float32)))
    src_v.copy_(torch.from_numpy(vp.astype(np.float32)))

    put_tab = rng.integers(-2, P + 2, size=nb).astype(np.int32)   # skips and repeats
    rb = hkv.record_bytes(fmt, tb, H)
    stride = (rb + 15) // 16 * 16 + 16 * int(rng.integers(0, 3))
    buf = torch.full((L, nb, stride), 0xA5, dtype=torch.uint8, device=DEV)
    rec = buf[:, :, :rb]

    if c["fused"]:
        crc_f = torch.zeros((L, nb), dtype=torch.int32, device=DEV)
        hkv.quant_crc(fmt, src_k, src_v, _i32(put_tab), rec, crc_out=crc_f)
    else:
        (hkv.quant_fp8 if fmt == "fp8" else hkv.quant_int4)(src_k, src_v, _i32(put_tab), rec)
    crc = hkv.crc32_blocks(rec, fmt, tb, H)
    torch.cuda.synchronize()

    ref, live = O.put(host_f64(src_k).astype(np.float32), host_f64(src_v).astype(np.float32),
                      put_tab, fmt)
    got = rec.cpu().numpy()
    for b in range(nb):
        if live[b]:
            assert np.array_equal(got[:, b], ref[:, b]), f"seed {seed}: record {b} differs"
        else:
            assert np.all(got[:, b] == 0xA5), f"seed {seed}: skipped record {b} was written"
    assert np.array_equal(crc_u32(crc), O.crc32_records(got)), f"seed {seed}: CRC differs"
    if c["fused"]:
        assert np.array_equal(crc_u32(crc_f)[:, live], O.crc32_records(ref)[:, live]), \
            f"seed {seed}: fused CRC differs"

    # fetch: a random subset of the live blocks onto distinct pages; others skipped
    cand = np.flatnonzero(live)
    take = cand[rng.random(len(cand)) < 0.8][:P]
    ftab = np.where(rng.random(nb) < 0.5, -1, P + rng.integers(0, 3, size=nb)).astype(np.int32)
    ftab[take] = rng.permutation(P)[:len(take)]
    span = int(rng.choice([50, 40000, 2 ** 31 - 1]))
    shape = (nb, tb) if c["per_token"] else (nb,)
    dm = rng.integers(-span, span, size=shape, endpoint=True).astype(np.int64)
    dm[rng.random(shape) < 0.2] = 0
    dm = np.clip(dm, -(2 ** 31), 2 ** 31 - 1).astype(np.int32)
    order = {"none": None,
             "page": hkv.page_visit_order(_i32(ftab), P),
             "random": _i32(rng.permutation(nb))}[c["order"]]
    out_k = canary_fill(_pages(L, P, tb, H, TORCH_OF[c["dst"]], rng))
    out_v = canary_fill(torch.empty_strided(out_k.shape, out_k.stride(), dtype=out_k.dtype,
                                            device=DEV))
    fetch = hkv.fetch_dequant_rope_shift_tokens if c["per_token"] else hkv.fetch_dequant_rope_shift
    fetch(rec, fmt, _i32(ftab), _i32(dm), c["base"], c["pairs"], out_k, out_v, visit_order=order)
    torch.cuda.synchronize()

    kr, vd = O.fetch_exact(ref, fmt, tb, H, dm, c["base"], c["pairs"])
    kd, _ = O.dequant_records(ref, fmt, tb, H)
    kg, vg = host_f64(out_k), host_f64(out_v)
    written = set()
    for b in take:
        page = int(ftab[b])
        written.add(page)
        what = f"seed {seed} block {b}"
        if c["per_token"]:
            check_values_exact(vg[:, page], O.round_output(vd[:, b], c["dst"]), f"{what} V")
            check_keys(kg[:, page], kr[:, b], kd[:, b], c["dst"], f"{what} K")
        else:
            compare_fetch_block(kg[:, page], vg[:, page], kr[:, b], vd[:, b], kd[:, b], c["dst"],
                                int(dm[b]), what)
    ck, cv = is_canary(out_k).cpu().numpy(), is_canary(out_v).cpu().numpy()
    for p in range(P):
        if p in written:
            assert not ck[:, p].any() and not cv[:, p].any(), f"seed {seed}: page {p} partly written"
        else:
            assert ck[:, p].all() and cv[:, p].all(), f"seed {seed}: page {p} was written"
