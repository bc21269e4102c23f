"""GPU parity of the frame container: put into frames, CRC, headers, a disk
round trip through the host, verification and fetch from frames, against the
CPU oracle.

Bar: frame bytes (header and record) bit-exact with the oracle's frames;
verification flags bit-exact with the oracle's on intact and tampered
frames; the per-block delta from the headers equal to the workload's; the
fetch from frames identical to the fetch from plain records."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from parity_util import TORCH_OF, crc_u32, host_f64
from quantization_rope_reuse_amd import hkv
from quantization_rope_reuse_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _host_pages(w, L):
    """Source pages [L, P, T_b, H, 128] (float32 values of the source dtype)
    with logical block b at page put_table[b]."""
    table = W.put_table(w)
    k = np.stack([W.pages_from_tokens(W.host_layer_values(w, l, 0), w, table) for l in range(L)])
    v = np.stack([W.pages_from_tokens(W.host_layer_values(w, l, 1), w, table) for l in range(L)])
    return k, v, table


def _build(w, fmt, L=None, layer_base=0, per_layer=False):
    """Put + CRC + headers on the GPU into fresh frames; returns
    (frames, oracle_frames, m_old, m_new, src_k, src_v)."""
    L = L or w.n_layers
    k, v, table = _host_pages(w, L)
    dt = TORCH_OF[w.src_dtype]
    kp = torch.from_numpy(k).to(DEV, dt)
    vp = torch.from_numpy(v).to(DEV, dt)
    tab = torch.from_numpy(table).to(DEV)
    m_old, m_new = W.block_positions(w)
    frames = hkv.alloc_frames(L, w.n_blocks, fmt, w.block_tokens, w.n_kv_heads, device=DEV)
    frames.fill_(0x5A)
    put = hkv.quant_fp8 if fmt == "fp8" else hkv.quant_int4
    mo = torch.from_numpy(m_old).to(DEV)
    if per_layer:
        for l in range(L):
            fl = frames[l:l + 1]
            put(kp[l:l + 1], vp[l:l + 1], tab, hkv.frame_records(fl))
            crc = hkv.crc32_blocks(hkv.frame_records(fl), fmt, w.block_tokens, w.n_kv_heads)
            hkv.frame_headers(fl, fmt, w.block_tokens, w.n_kv_heads, crc, mo,
                              layer_base=layer_base + l)
    else:
        put(kp, vp, tab, hkv.frame_records(frames))
        crc = hkv.crc32_blocks(hkv.frame_records(frames), fmt, w.block_tokens, w.n_kv_heads)
        hkv.frame_headers(frames, fmt, w.block_tokens, w.n_kv_heads, crc, mo,
                          layer_base=layer_base)
    torch.cuda.synchronize()
    # the oracle sees the values as the GPU did (after the dtype cast)
    rec, _ = O.put(host_f64(kp).astype(np.float32), host_f64(vp).astype(np.float32), table, fmt)
    ref = O.make_frames(rec, fmt, w.block_tokens, w.n_kv_heads, m_old, layer_base=layer_base)
    return frames, ref, m_old, m_new, kp, vp


def _fetch(records, fmt, w, dm, L):
    dt = TORCH_OF[w.out_dtype]
    ftab = torch.from_numpy(W.fetch_table(w)).to(DEV)
    shape = (L, int(ftab.max()) + 1, w.block_tokens, w.n_kv_heads, 128)
    ok = torch.zeros(shape, dtype=dt, device=DEV)
    ov = torch.zeros(shape, dtype=dt, device=DEV)
    hkv.fetch_dequant_rope_shift(records, fmt, ftab, dm, w.rope_base, w.pairs, ok, ov)
    return ok, ov


@pytest.mark.parametrize("fmt", ["fp8", "int4"])
def test_gqa_frames_bit_exact_and_fetch(fmt):
    w = W.GQA_REORDER
    print(f"[frames] {w.name} {fmt}", flush=True)
    frames, ref, m_old, m_new, _, _ = _build(w, fmt, layer_base=7)
    got = frames.cpu().numpy()
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} frame bytes differ"
    flags = hkv.frame_verify(frames, fmt, w.block_tokens, w.n_kv_heads, layer_base=7)
    assert not flags.cpu().numpy().any()
    dm = hkv.frame_delta_m(frames, fmt, w.block_tokens, w.n_kv_heads,
                           torch.from_numpy(m_new).to(DEV))
    assert np.array_equal(dm.cpu().numpy(), W.delta_m(w))
    # fetch from the frames equals fetch from a plain copy of the records
    plain = hkv.alloc_records(w.n_layers, w.n_blocks, fmt, w.block_tokens, w.n_kv_heads,
                              device=DEV)
    plain.copy_(hkv.frame_records(frames))
    a = _fetch(hkv.frame_records(frames), fmt, w, dm, w.n_layers)
    b = _fetch(plain, fmt, w, dm, w.n_layers)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_disk_round_trip_and_tamper(tmp_path):
    w = W.GQA_REORDER
    fmt = "int4"
    print(f"[frames] disk round trip {w.name}", flush=True)
    frames, ref, m_old, m_new, _, _ = _build(w, fmt, L=2)
    L, nb, fb = frames.shape
    # to the host, to a file of packed frames, back into a fresh device buffer
    path = tmp_path / "cache.hkvf"
    frames.cpu().numpy().reshape(L * nb, fb).tofile(path)
    assert path.stat().st_size == L * nb * fb
    disk = np.fromfile(path, dtype=np.uint8).reshape(L, nb, fb)
    assert np.array_equal(disk, ref)
    back = hkv.alloc_frames(L, nb, fmt, w.block_tokens, w.n_kv_heads, device=DEV)
    back.copy_(torch.from_numpy(disk))
    assert not hkv.frame_verify(back, fmt, w.block_tokens, w.n_kv_heads).cpu().numpy().any()
    dm = hkv.frame_delta_m(back, fmt, w.block_tokens, w.n_kv_heads,
                           torch.from_numpy(m_new).to(DEV))
    a = _fetch(hkv.frame_records(back), fmt, w, dm, L)
    b = _fetch(hkv.frame_records(frames), fmt, w, dm, L)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])

    # damage in the file: the GPU's flags equal the oracle's
    rng = np.random.default_rng(5)
    t = disk.copy()
    t[0, 3, 1] ^= 0x04                                   # magic
    t[1, 10, 13] ^= 0x01                                 # block_tokens field
    t[0, 20, 61] ^= 0x80                                 # stored header CRC
    for _ in range(5):                                   # payload bits
        l, b, j = int(rng.integers(L)), int(rng.integers(nb)), int(rng.integers(64, fb))
        t[l, b, j] ^= np.uint8(1 << int(rng.integers(8)))
    t[1, [40, 41]] = t[1, [41, 40]]                      # swapped frames
    back.copy_(torch.from_numpy(t))
    got = hkv.frame_verify(back, fmt, w.block_tokens, w.n_kv_heads).cpu().numpy()
    want = O.verify_frames(t, fmt, w.block_tokens, w.n_kv_heads).astype(np.int64)
    assert np.array_equal(got.astype(np.int64) & 0xFFFFFFFF, want)
    assert want[0, 3] & O.FRAME_BAD_MAGIC and want[1, 40] & O.FRAME_BAD_INDEX
    assert np.count_nonzero(want) >= 5
    # a wrong shape or layer base flags every frame; FP8 frames would not fit
    # this buffer, which the binding rejects before any library call
    bad_geo = hkv.frame_verify(back, fmt, w.block_tokens // 2, w.n_kv_heads).cpu().numpy()
    assert (bad_geo & O.FRAME_BAD_GEOMETRY).all()
    with pytest.raises(ValueError, match="needs"):
        hkv.frame_verify(back, "fp8", w.block_tokens, w.n_kv_heads)
    bad_layer = hkv.frame_verify(back, fmt, w.block_tokens, w.n_kv_heads,
                                 layer_base=1).cpu().numpy()
    assert (bad_layer & O.FRAME_BAD_INDEX).all()


def test_per_layer_headers_and_padded_frames():
    # one call per layer with its own layer_base, frames padded to a 16-byte
    # stride larger than header + record (odd head count -> ragged record)
    w = W.KVWorkload(name="frames_ragged", n_layers=3, n_kv_heads=3, n_tokens=50,
                     block_tokens=7, src_dtype="bf16", out_dtype="f16", rope_base=1e4,
                     pairs="interleaved", formats=("fp8",), delta_kind="uniform",
                     delta_value=3000)
    print(f"[frames] {w.name}", flush=True)
    frames, ref, m_old, m_new, _, _ = _build(w, "fp8", layer_base=100, per_layer=True)
    assert frames.stride(1) > frames.shape[2]            # padded
    got = frames.cpu().numpy()
    assert np.array_equal(got, ref)
    flags = hkv.frame_verify(frames, "fp8", w.block_tokens, w.n_kv_heads, layer_base=100)
    assert not flags.cpu().numpy().any()
    dm = hkv.frame_delta_m(frames, "fp8", w.block_tokens, w.n_kv_heads,
                           torch.from_numpy(m_new).to(DEV)).cpu().numpy()
    assert np.array_equal(dm, W.delta_m(w))
    # extreme positions clamp to the int32 range
    mo = torch.tensor([-2**31] + [0] * (w.n_blocks - 1), dtype=torch.int32, device=DEV)
    crc = hkv.crc32_blocks(hkv.frame_records(frames[:1]), "fp8", w.block_tokens, w.n_kv_heads)
    hkv.frame_headers(frames[:1], "fp8", w.block_tokens, w.n_kv_heads, crc, mo, layer_base=100)
    mn = torch.tensor([2**31 - 1] + [5] * (w.n_blocks - 1), dtype=torch.int32, device=DEV)
    d = hkv.frame_delta_m(frames[:1], "fp8", w.block_tokens, w.n_kv_heads, mn).cpu().numpy()
    assert d[0] == 2**31 - 1 and (d[1:] == 5).all()


def test_int4_l3_full_size_frames():
    w = W.INT4_L3
    print(f"[frames] full {w.name}", flush=True)
    L, nb = w.n_layers, w.n_blocks
    dt = TORCH_OF[w.src_dtype]
    shape = (L, nb, w.block_tokens, w.n_kv_heads, 128)
    kp = torch.empty(shape, dtype=dt, device=DEV)
    vp = torch.empty_like(kp)
    tab = torch.from_numpy(W.put_table(w)).to(DEV)
    tmp = torch.empty((w.n_tokens, w.n_kv_heads, 128), dtype=torch.float32, device=DEV)
    gen = torch.Generator(device=DEV)
    for l in range(L):
        for kv, dst in ((0, kp), (1, vp)):
            W.device_layer_values(w, l, kv, tmp, generator=gen)
            dst[l].index_copy_(0, tab.long(), tmp.view(nb, w.block_tokens, w.n_kv_heads,
                                                        128).to(dt))
    m_old, m_new = W.block_positions(w)
    frames = hkv.alloc_frames(L, nb, "int4", w.block_tokens, w.n_kv_heads, device=DEV)
    hkv.quant_int4(kp, vp, tab, hkv.frame_records(frames))
    crc = hkv.crc32_blocks(hkv.frame_records(frames), "int4", w.block_tokens, w.n_kv_heads)
    hkv.frame_headers(frames, "int4", w.block_tokens, w.n_kv_heads, crc,
                      torch.from_numpy(m_old).to(DEV))
    flags = hkv.frame_verify(frames, "int4", w.block_tokens, w.n_kv_heads)
    torch.cuda.synchronize()
    assert not flags.cpu().numpy().any()
    # sampled frames against the oracle
    rng = np.random.default_rng(31)
    crc_np = crc_u32(crc)
    for l, b in [(0, 0), (L - 1, nb - 1)] + [(int(rng.integers(L)), int(rng.integers(nb)))
                                             for _ in range(6)]:
        got = frames[l, b].cpu().numpy()
        page = int(W.put_table(w)[b])
        xk = host_f64(kp[l, page]).astype(np.float32)
        xv = host_f64(vp[l, page]).astype(np.float32)
        kc, ks = O.quant_int4_vectors(xk)
        vc, vs = O.quant_int4_vectors(xv)
        rec = O.assemble_records(kc, vc, ks, vs)
        assert int(O.crc32_records(rec[None])[0]) == int(crc_np[l, b])
        want = np.concatenate([O.frame_header("int4", w.block_tokens, w.n_kv_heads, l, b,
                                              int(m_old[b]), rec.size, int(crc_np[l, b])), rec])
        assert np.array_equal(got, want), (l, b)
    # flip one payload bit in a few frames: exactly those are flagged
    for trial in range(3):
        l, b = int(rng.integers(L)), int(rng.integers(nb))
        j = 64 + int(rng.integers(frames.shape[2] - 64))
        frames[l, b, j] ^= 1
        f = hkv.frame_verify(frames, "int4", w.block_tokens, w.n_kv_heads).cpu().numpy()
        assert np.argwhere(f).tolist() == [[l, b]] and f[l, b] == O.FRAME_BAD_PAYLOAD_CRC
        frames[l, b, j] ^= 1
