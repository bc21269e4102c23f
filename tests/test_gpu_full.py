"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses: the Qwen3-8B-shaped cache (36 layers, 32k tokens, fp16, one
call per operation), the Llama-3-70B-shaped cache (80 layers, 64k tokens,
bf16, fetch layer by layer on a side stream) and the INT4 disk-tier cache
(32 layers, 16k tokens, fp16 with outlier channels, CRC tamper test, and the
put and CRC in one pass against the two passes).

Three levels of checking:
* one whole layer (seeded choice) against the oracle element by element:
  every record byte and CRC, every V value exact, every key within the
  tolerance (exact where the block's delta is 0);
* sampled blocks of other layers (seeded, plus the blocks with the extreme
  deltas and the first and last block) the same way;
* the whole cache on the device, with no oracle, by properties that hold at
  any size: records decoded with the format's definition (an E4M3 table,
  INT4 nibbles) times their scales, rounded to the page dtype, equal every V
  page and every key page of a zero-delta block; rotated key vectors keep
  the norm of their decoded vector within the output rounding; every source
  element lies within half a code step of its decoded value (FP8: 2^-4 of
  |x| plus 2^-10 s; INT4: s / 2); every page written; the CRC kernel agrees
  with the CRCs the put wrote."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from parity_util import (TORCH_OF, canary_fill, check_keys, check_values_exact, crc_u32,
                         host_f64, is_canary)
from quantization_rope_reuse_amd import hkv
from quantization_rope_reuse_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _fill_source(w, L=None):
    """Source pages [L, P, T_b, H, 128] of the workload's dtype, logical block
    b of each layer stored at page put_table[b]."""
    L = L or w.n_layers
    nb, tb, H = w.n_blocks, w.block_tokens, w.n_kv_heads
    dt = TORCH_OF[w.src_dtype]
    k = torch.empty((L, nb, tb, H, 128), dtype=dt, device=DEV)
    v = torch.empty_like(k)
    put_tab = torch.from_numpy(W.put_table(w)).to(DEV)
    tmp = torch.empty((w.n_tokens, H, 128), dtype=torch.float32, device=DEV)
    gen = torch.Generator(device=DEV)
    for l in range(L):
        for kv, dst in ((0, k), (1, v)):
            W.device_layer_values(w, l, kv, tmp, generator=gen)
            dst[l].index_copy_(0, put_tab.long(), tmp.view(nb, tb, H, 128).to(dt))
    return k, v, put_tab


def _samples(w, L, rng, n):
    dm = W.delta_m(w)
    blocks = {0, w.n_blocks - 1, int(np.argmax(dm)), int(np.argmin(dm))}
    while len(blocks) < n:
        blocks.add(int(rng.integers(w.n_blocks)))
    layers = [0, L - 1] + [int(x) for x in rng.integers(0, L, size=n)]
    return [(layers[i % len(layers)], b) for i, b in enumerate(sorted(blocks))]


def _check_block(w, fmt, l, b, src_k, src_v, put_tab, rec, crc, out_k, out_v, ftab, dm):
    """Oracle on one (layer, block) against the GPU's record, CRC and pages."""
    page_src = int(put_tab[b])
    xk = host_f64(src_k[l, page_src]).astype(np.float32)       # [T_b, H, 128]
    xv = host_f64(src_v[l, page_src]).astype(np.float32)
    quant = O.quant_fp8_vectors if fmt == "fp8" else O.quant_int4_vectors
    kc, ks = quant(xk)
    vc, vs = quant(xv)
    ref = O.assemble_records(kc, vc, ks, vs)
    got = rec[l, b].cpu().numpy()
    assert np.array_equal(got, ref), f"layer {l} block {b}: {np.count_nonzero(got != ref)} bytes"
    assert int(crc_u32(crc[l, b:b + 1])[0]) == int(O.crc32_records(ref[None])[0])
    kd, vd = O.dequant_records(ref, fmt, w.block_tokens, w.n_kv_heads)
    kr = O.rope_shift(kd, float(dm[b]), w.rope_base, w.pairs)
    page = int(ftab[b])
    kg = host_f64(out_k[l, page])
    vg = host_f64(out_v[l, page])
    check_values_exact(vg, O.round_output(vd, w.out_dtype), f"layer {l} block {b} V")
    if dm[b] == 0:
        check_values_exact(kg, O.round_output(kd, w.out_dtype), f"layer {l} block {b} K")
    else:
        check_keys(kg, kr, kd, w.out_dtype, f"layer {l} block {b} K")


def _check_layer(w, fmt, l, src_k, src_v, put_np, rec, crc, out_k, out_v, ftab_np, dm_np,
                 chunk=128):
    """Every block of layer l against the oracle, chunk blocks at a time."""
    nb, tb, H = w.n_blocks, w.block_tokens, w.n_kv_heads
    quant = O.quant_fp8_vectors if fmt == "fp8" else O.quant_int4_vectors
    worst = 0.0
    for b0 in range(0, nb, chunk):
        bs = np.arange(b0, min(nb, b0 + chunk))
        src_pages = torch.from_numpy(put_np[bs]).long().to(DEV)
        xk = host_f64(src_k[l].index_select(0, src_pages)).astype(np.float32)
        xv = host_f64(src_v[l].index_select(0, src_pages)).astype(np.float32)
        kc, ks = quant(xk)
        vc, vs = quant(xv)
        ref = O.assemble_records(kc, vc, ks, vs)                 # [n, rb]
        got = rec[l, b0:b0 + bs.size].cpu().numpy()
        bad = got != ref
        assert not bad.any(), f"layer {l} blocks {b0}..: {int(bad.sum())} record bytes differ"
        assert np.array_equal(crc_u32(crc[l, b0:b0 + bs.size]), O.crc32_records(ref)), \
            f"layer {l} blocks {b0}..: CRC"
        kd, vd = O.dequant_records(ref, fmt, tb, H)               # [n, T_b, H, 128]
        dst_pages = torch.from_numpy(ftab_np[bs]).long().to(DEV)
        kg = host_f64(out_k[l].index_select(0, dst_pages))
        vg = host_f64(out_v[l].index_select(0, dst_pages))
        check_values_exact(vg, O.round_output(vd, w.out_dtype), f"layer {l} blocks {b0}.. V")
        dm = dm_np[bs]
        zero = dm == 0
        if zero.any():
            check_values_exact(kg[zero], O.round_output(kd[zero], w.out_dtype),
                               f"layer {l} blocks {b0}.. K (dm = 0)")
        if (~zero).any():
            kr = O.rope_shift(kd[~zero], dm[~zero].astype(np.float64)[:, None, None],
                              w.rope_base, w.pairs)
            worst = max(worst, check_keys(kg[~zero], kr, kd[~zero], w.out_dtype,
                                          f"layer {l} blocks {b0}.. K"))
        del xk, xv, kd, vd, kg, vg
    return worst


def _e4m3_table():
    """Decoded value of each of the 256 E4M3FN codes (bias 7, 3 mantissa
    bits, subnormals m/8 * 2^-6, 0x7F / 0xFF NaN), from the format's
    definition, as an fp32 device tensor."""
    c = np.arange(256)
    e, m = (c >> 3) & 15, c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7))
    val = np.where(c >= 128, -mag, mag)
    val[(c & 0x7F) == 0x7F] = np.nan
    return torch.tensor(val, dtype=torch.float32, device=DEV)


def _decode_layer(rec_l, fmt, vecs):
    """Records of one layer [nb, >= rb] -> decoded K, V [nb, vecs, 128] fp32
    (code times scale, exact in fp32) and the scales [nb, vecs]."""
    cb = 128 if fmt == "fp8" else 64
    n = vecs * cb
    scales = rec_l[:, 2 * n:2 * n + 4 * vecs].contiguous().view(torch.float16).float()
    ks, vs = scales[:, :vecs], scales[:, vecs:]
    out = []
    for part, s in ((rec_l[:, :n], ks), (rec_l[:, n:2 * n], vs)):
        codes = part.reshape(-1, vecs, cb)
        if fmt == "fp8":
            vals = _e4m3_table()[codes.long()]
        else:
            c = codes.to(torch.int16)
            lo = ((c & 0xF) ^ 8) - 8                               # two's complement nibble
            hi = ((c >> 4) ^ 8) - 8
            vals = torch.stack([lo, hi], dim=-1).reshape(-1, vecs, 128).float()
        out.append(vals * s[..., None])
    return out[0], out[1], ks, vs


def _whole_cache(w, fmt, rec, src_k, src_v, put_tab, out_k, out_v, ftab, dm, crc):
    """Properties over every layer and block, on the device (no oracle).
    dm: device int32 [n_blocks], zero for the blocks whose keys are not
    rotated; crc: the CRCs written with the records, or None."""
    nb, tb, H = w.n_blocks, w.block_tokens, w.n_kv_heads
    vecs = tb * H
    odt = out_k.dtype
    # relative half-ulp of the page dtype, and its smallest spacing
    rel = {torch.float32: 2.0 ** -24, torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}[odt]
    tiny = {torch.float32: 2.0 ** -149, torch.float16: 2.0 ** -24, torch.bfloat16: 2.0 ** -133}[odt]
    if crc is not None:
        crc2 = hkv.crc32_blocks(rec, fmt, tb, H)
        assert torch.equal(crc2, crc), "the CRC kernel disagrees with the CRCs of the put"
    zero = (dm == 0)
    put_l, f_l = put_tab.long(), ftab.long()
    for l in range(src_k.shape[0]):
        kd, vd, ks, vs = _decode_layer(rec[l], fmt, vecs)
        ok = out_k[l].index_select(0, f_l).reshape(nb, vecs, 128)
        ov = out_v[l].index_select(0, f_l).reshape(nb, vecs, 128)
        assert not bool(is_canary(ok).any()) and not bool(is_canary(ov).any()), \
            f"layer {l}: a page was not written"
        assert bool((ov == vd.to(odt)).all()), f"layer {l}: V differs from code * scale"
        if bool(zero.any()):
            assert bool((ok[zero] == kd[zero].to(odt)).all()), \
                f"layer {l}: a zero-delta key differs from code * scale"
        # rotation keeps the norm up to the fp32 rotation error (2e-6 of the
        # norm per element) and the output rounding (half an ulp per element)
        okf = ok.float()
        n_out = okf.norm(dim=-1)
        n_deq = kd.norm(dim=-1)
        tol = rel * n_out + 128 ** 0.5 * (2e-6 * n_deq + tiny)
        assert bool(((n_out - n_deq).abs() <= tol).all()), f"layer {l}: key norm not kept"
        # each source element within half a code step of its decoded value
        for src, deq, s in ((src_k, kd, ks), (src_v, vd, vs)):
            x = src[l].index_select(0, put_l).reshape(nb, vecs, 128).float()
            err = (x - deq).abs()
            if fmt == "fp8":
                lim = 2.0 ** -4 * x.abs() * (1 + 2.0 ** -16) + 2.0 ** -10 * s[..., None]
            else:
                lim = 0.5 * s[..., None] * (1 + 2.0 ** -16)
            assert bool((err <= lim).all()), \
                f"layer {l}: a source element is beyond half a code step ({float((err - lim).max())})"
            del x, err, lim
        del kd, vd, ok, ov, okf


def _whole_layer_and_samples(w, fmt, rng, src_k, src_v, put_tab, rec, crc, out_k, out_v, ftab,
                             dm_np):
    """One seeded layer in full, then sampled blocks of the other layers,
    against the oracle."""
    L = src_k.shape[0]
    put_np, ftab_np = put_tab.cpu().numpy(), ftab.cpu().numpy()
    layer = int(rng.integers(L))
    print(f"[full] {w.name}: layer {layer} against the oracle", flush=True)
    _check_layer(w, fmt, layer, src_k, src_v, put_np, rec, crc, out_k, out_v, ftab_np, dm_np)
    for l, b in _samples(w, L, rng, 8):
        if l != layer:
            _check_block(w, fmt, l, b, src_k, src_v, put_np, rec, crc, out_k, out_v, ftab_np,
                         dm_np)


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_qwen3_8b_full():
    w = W.QWEN3_8B
    print(f"[full] {w.name}", flush=True)
    src_k, src_v, put_tab = _fill_source(w)
    L, nb = w.n_layers, w.n_blocks
    rec = hkv.alloc_records(L, nb, "fp8", w.block_tokens, w.n_kv_heads, device=DEV)
    hkv.quant_fp8(src_k, src_v, put_tab, rec)
    crc = hkv.crc32_blocks(rec, "fp8", w.block_tokens, w.n_kv_heads)
    ftab = torch.from_numpy(W.fetch_table(w)).to(DEV)
    dm_np = W.delta_m(w)
    dm = torch.from_numpy(dm_np).to(DEV)
    out_k = canary_fill(torch.empty_like(src_k))
    out_v = canary_fill(torch.empty_like(src_v))
    order = hkv.page_visit_order(ftab, nb)
    hkv.fetch_dequant_rope_shift(rec, "fp8", ftab, dm, w.rope_base, w.pairs, out_k, out_v,
                                 visit_order=order)
    torch.cuda.synchronize()
    rng = np.random.default_rng(81)
    _whole_layer_and_samples(w, "fp8", rng, src_k, src_v, put_tab, rec, crc, out_k, out_v,
                             ftab, dm_np)
    _whole_cache(w, "fp8", rec, src_k, src_v, put_tab, out_k, out_v, ftab, dm, crc)


def test_llama3_70b_full_layerwise_side_stream():
    w = W.LLAMA3_70B
    print(f"[full] {w.name}", flush=True)
    src_k, src_v, put_tab = _fill_source(w)
    L, nb = w.n_layers, w.n_blocks
    rec = hkv.alloc_records(L, nb, "fp8", w.block_tokens, w.n_kv_heads, device=DEV)
    # put and CRC in one pass, as the benchmark step runs them
    crc = hkv.quant_crc("fp8", src_k, src_v, put_tab, rec)
    ftab = torch.from_numpy(W.fetch_table(w)).to(DEV)
    dm_np = W.delta_m(w)
    dm = torch.from_numpy(dm_np).to(DEV)
    out_k = canary_fill(torch.empty_like(src_k))
    out_v = canary_fill(torch.empty_like(src_v))
    side = torch.cuda.Stream()
    ready = torch.cuda.Event()
    ready.record(torch.cuda.current_stream())
    side.wait_event(ready)
    order = hkv.page_visit_order(ftab, nb, stream=side)
    for l in range(L):
        hkv.fetch_dequant_rope_shift(rec[l:l + 1], "fp8", ftab, dm, w.rope_base, w.pairs,
                                     out_k[l:l + 1], out_v[l:l + 1], visit_order=order,
                                     stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    rng = np.random.default_rng(82)
    _whole_layer_and_samples(w, "fp8", rng, src_k, src_v, put_tab, rec, crc, out_k, out_v,
                             ftab, dm_np)
    _whole_cache(w, "fp8", rec, src_k, src_v, put_tab, out_k, out_v, ftab, dm, crc)


def test_llama3_70b_staged_full():
    """The layer-wise staged fetch at full size: all 80 layers' records (from
    the fused put) in pinned host memory, copied layer by layer into two
    staging buffers and fetched on separate copy and fetch streams, with the
    benchmark's table, deltas and visit order.  Every layer's pages equal,
    byte for byte, a fetch of the same layer from device memory (whose
    parity at this size the test above checks), so no staging buffer was
    refilled before its fetch had read it; every layer's ready event was
    recorded."""
    w = W.LLAMA3_70B
    print(f"[full] {w.name} staged", flush=True)
    src_k, src_v, put_tab = _fill_source(w)
    L, nb, tb, H = w.n_layers, w.n_blocks, w.block_tokens, w.n_kv_heads
    rec = hkv.alloc_records(L, nb, "fp8", tb, H, device=DEV)
    hkv.quant_crc("fp8", src_k, src_v, put_tab, rec)
    del src_k, src_v
    torch.cuda.synchronize()
    host = torch.empty(rec.shape, dtype=torch.uint8, pin_memory=True)
    host.copy_(rec)
    print(f"[full] {host.numel() / 1e9:.2f} GB of records pinned", flush=True)
    ftab = torch.from_numpy(W.fetch_table(w)).to(DEV)
    dm = torch.from_numpy(W.delta_m(w)).to(DEV)
    order = hkv.page_visit_order(ftab, nb)
    out_k = canary_fill(torch.empty((L, nb, tb, H, 128), dtype=torch.bfloat16, device=DEV))
    out_v = canary_fill(torch.empty_like(out_k))
    staging = hkv.alloc_staging(nb, "fp8", tb, H, device=DEV)
    copy_s, fetch_s = torch.cuda.Stream(), torch.cuda.Stream()
    ready = [torch.cuda.Event() for _ in range(L)]
    torch.cuda.synchronize()
    hkv.fetch_staged(host[:, :, :hkv.record_bytes("fp8", tb, H)], "fp8", ftab, dm, w.rope_base,
                     w.pairs, out_k, out_v, staging, visit_order=order, copy_stream=copy_s,
                     fetch_stream=fetch_s, layer_ready=ready)
    fetch_s.synchronize()
    assert all(e.query() for e in ready)
    torch.cuda.synchronize()
    ok = torch.empty_like(out_k[:1])
    ov = torch.empty_like(out_v[:1])
    for l in range(L):
        hkv.fetch_dequant_rope_shift(rec[l:l + 1], "fp8", ftab, dm, w.rope_base, w.pairs, ok, ov,
                                     visit_order=order)
        assert torch.equal(ok[0].view(torch.uint8), out_k[l].view(torch.uint8)), f"K layer {l}"
        assert torch.equal(ov[0].view(torch.uint8), out_v[l].view(torch.uint8)), f"V layer {l}"
    print(f"[full] {L} staged layers equal the device-memory fetch", flush=True)


def test_llama3_70b_per_token_deltas_full():
    """The per-token fetch at the Llama-3-70B shape in the benchmark's launch
    configuration (one layer per launch on a side stream, blocks in page
    order), with random deltas per token (some blocks all zero): sampled
    blocks against the oracle, the whole cache by its properties."""
    w = W.LLAMA3_70B
    print(f"[full] {w.name} per-token deltas", flush=True)
    src_k, src_v, put_tab = _fill_source(w)
    L, nb, tb, H = w.n_layers, w.n_blocks, w.block_tokens, w.n_kv_heads
    rec = hkv.alloc_records(L, nb, "fp8", tb, H, device=DEV)
    hkv.quant_crc("fp8", src_k, src_v, put_tab, rec)
    rng = np.random.default_rng(86)
    dmt = rng.integers(-(1 << 20), 1 << 20, size=(nb, tb)).astype(np.int32)
    zero_blocks = rng.choice(nb, size=4, replace=False)
    dmt[zero_blocks] = 0
    ftab_np = W.fetch_table(w)
    ftab = torch.from_numpy(ftab_np).to(DEV)
    dmt_dev = torch.from_numpy(dmt).to(DEV)
    out_k = canary_fill(torch.empty_like(src_k))
    out_v = canary_fill(torch.empty_like(src_v))
    side = torch.cuda.Stream()
    ready = torch.cuda.Event()
    ready.record(torch.cuda.current_stream())
    side.wait_event(ready)
    order = hkv.page_visit_order(ftab, nb, stream=side)
    for l in range(L):
        hkv.fetch_dequant_rope_shift_tokens(rec[l:l + 1], "fp8", ftab, dmt_dev, w.rope_base,
                                            w.pairs, out_k[l:l + 1], out_v[l:l + 1],
                                            visit_order=order, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    put_np = put_tab.cpu().numpy()
    blocks = sorted(set(int(b) for b in rng.choice(nb, size=6, replace=False)) |
                    {int(zero_blocks[0]), 0, nb - 1})
    for i, b in enumerate(blocks):
        l = [0, L - 1, int(rng.integers(L))][i % 3]
        xk = host_f64(src_k[l, int(put_np[b])]).astype(np.float32)
        xv = host_f64(src_v[l, int(put_np[b])]).astype(np.float32)
        kc, ks = O.quant_fp8_vectors(xk)
        vc, vs = O.quant_fp8_vectors(xv)
        ref = O.assemble_records(kc, vc, ks, vs)
        assert np.array_equal(rec[l, b].cpu().numpy(), ref), f"layer {l} block {b} record"
        kr, vd = O.fetch_exact(ref[None, None], "fp8", tb, H, dmt[b:b + 1], w.rope_base, w.pairs)
        kd, _ = O.dequant_records(ref[None, None], "fp8", tb, H)
        page = int(ftab_np[b])
        kg = host_f64(out_k[l, page])
        vg = host_f64(out_v[l, page])
        check_values_exact(vg, O.round_output(vd[0, 0], w.out_dtype), f"layer {l} block {b} V")
        if not dmt[b].any():
            check_values_exact(kg, O.round_output(kd[0, 0], w.out_dtype), f"layer {l} block {b} K")
        else:
            check_keys(kg, kr[0, 0], kd[0, 0], w.out_dtype, f"layer {l} block {b} K")
    rotated = torch.from_numpy(dmt.any(axis=1).astype(np.int32)).to(DEV)
    _whole_cache(w, "fp8", rec, src_k, src_v, put_tab, out_k, out_v, ftab, rotated, None)


def test_llama3_70b_tp8_shard():
    """One GPU's tensor-parallel share of the Llama-3-70B-shaped cache: one KV
    head, 64 vectors per block (two 32-vector fetch chunks, one fused put
    chunk).  Put and CRC in one pass, 80 per-layer fetches on a side stream,
    the same checks as the full cache."""
    w = W.LLAMA3_70B_TP8
    print(f"[full] {w.name}", flush=True)
    src_k, src_v, put_tab = _fill_source(w)
    L, nb = w.n_layers, w.n_blocks
    rec = hkv.alloc_records(L, nb, "fp8", w.block_tokens, w.n_kv_heads, device=DEV)
    crc = hkv.quant_crc("fp8", src_k, src_v, put_tab, rec)
    ftab = torch.from_numpy(W.fetch_table(w)).to(DEV)
    dm_np = W.delta_m(w)
    dm = torch.from_numpy(dm_np).to(DEV)
    out_k = canary_fill(torch.empty_like(src_k))
    out_v = canary_fill(torch.empty_like(src_v))
    side = torch.cuda.Stream()
    ready = torch.cuda.Event()
    ready.record(torch.cuda.current_stream())
    side.wait_event(ready)
    order = hkv.page_visit_order(ftab, nb, stream=side)
    for l in range(L):
        hkv.fetch_dequant_rope_shift(rec[l:l + 1], "fp8", ftab, dm, w.rope_base, w.pairs,
                                     out_k[l:l + 1], out_v[l:l + 1], visit_order=order,
                                     stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    rng = np.random.default_rng(84)
    _whole_layer_and_samples(w, "fp8", rng, src_k, src_v, put_tab, rec, crc, out_k, out_v,
                             ftab, dm_np)
    _whole_cache(w, "fp8", rec, src_k, src_v, put_tab, out_k, out_v, ftab, dm, crc)


def test_int4_l3_full_with_tamper():
    w = W.INT4_L3
    print(f"[full] {w.name}", flush=True)
    src_k, src_v, put_tab = _fill_source(w)
    L, nb = w.n_layers, w.n_blocks
    rec = hkv.alloc_records(L, nb, "int4", w.block_tokens, w.n_kv_heads, device=DEV)
    hkv.quant_int4(src_k, src_v, put_tab, rec)
    crc = hkv.crc32_blocks(rec, "int4", w.block_tokens, w.n_kv_heads)
    ftab = torch.from_numpy(W.fetch_table(w)).to(DEV)
    dm_np = W.delta_m(w)
    dm = torch.from_numpy(dm_np).to(DEV)
    out_k = canary_fill(torch.empty_like(src_k))
    out_v = canary_fill(torch.empty_like(src_v))
    hkv.fetch_dequant_rope_shift(rec, "int4", ftab, dm, w.rope_base, w.pairs, out_k, out_v)
    torch.cuda.synchronize()
    rng = np.random.default_rng(83)
    _whole_layer_and_samples(w, "int4", rng, src_k, src_v, put_tab, rec, crc, out_k, out_v,
                             ftab, dm_np)
    _whole_cache(w, "int4", rec, src_k, src_v, put_tab, out_k, out_v, ftab, dm, crc)

    # put and CRC in one pass: the same records and the same CRCs
    rec2 = hkv.alloc_records(L, nb, "int4", w.block_tokens, w.n_kv_heads, device=DEV)
    crc2 = hkv.quant_crc("int4", src_k, src_v, put_tab, rec2)
    torch.cuda.synchronize()
    assert torch.equal(rec2, rec) and torch.equal(crc2, crc)
    del rec2

    # tamper detection: flip single bits / bytes in a few records; exactly
    # those records' CRCs change, to the oracle's CRC of the tampered bytes
    base_crc = crc_u32(crc)
    for trial in range(4):
        l, b = int(rng.integers(L)), int(rng.integers(nb))
        j = int(rng.integers(rec.shape[2]))
        mask = int(1 << rng.integers(8)) if trial % 2 == 0 else 0xFF
        rec[l, b, j] ^= mask
        new = crc_u32(hkv.crc32_blocks(rec, "int4", w.block_tokens, w.n_kv_heads))
        diff = np.argwhere(new != base_crc)
        assert diff.tolist() == [[l, b]], (trial, diff.tolist())
        assert int(new[l, b]) == int(O.crc32_records(rec[l, b].cpu().numpy()[None])[0])
        rec[l, b, j] ^= mask
    again = crc_u32(hkv.crc32_blocks(rec, "int4", w.block_tokens, w.n_kv_heads))
    assert np.array_equal(again, base_crc)
