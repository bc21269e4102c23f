"""Layer-wise staged fetch (hkv_fetch_staged) against the oracle.

Records written by the oracle sit in pinned host memory; the library copies
them layer by layer into two device staging buffers on a copy stream and
fetches each layer from there on a fetch stream, while a compute stream
waits on each layer's ready event and snapshots that layer's pages (plus a
matrix product standing in for the suffix compute).  Checked:
* every layer's pages against the oracle (V and zero-delta keys exact, other
  keys within the fetch tolerance), so no staging buffer was refilled before
  its fetch had read it;
* the snapshots the compute stream took right after each ready event equal
  the final pages, so the events are recorded after the layer's fetch;
* the pages equal a plain fetch of the same records from device memory."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from parity_util import TORCH_OF, canary_fill, check_keys, check_values_exact, host_f64
from quantization_rope_reuse_amd import hkv

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _oracle_records(L, nb, tb, H, fmt, src_dtype, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((L, nb, tb, H, 128)).astype(np.float32)
    v = rng.standard_normal((L, nb, tb, H, 128)).astype(np.float32)
    # the source dtype's values, as an engine would hold them
    k = host_f64(torch.from_numpy(k).to(TORCH_OF[src_dtype])).astype(np.float32)
    v = host_f64(torch.from_numpy(v).to(TORCH_OF[src_dtype])).astype(np.float32)
    ref, _ = O.put(k, v, np.arange(nb), fmt)
    return ref


def _run(L, nb, tb, H, fmt, src_dtype, out_dtype, pairs, base, seed, separate_streams):
    rng = np.random.default_rng(seed + 1)
    ref = _oracle_records(L, nb, tb, H, fmt, src_dtype, seed)
    rb = ref.shape[2]
    stride = (rb + 15) // 16 * 16
    host = torch.zeros((L, nb, stride), dtype=torch.uint8).pin_memory()
    host[:, :, :rb] = torch.from_numpy(ref)
    host_rec = host[:, :, :rb]
    table = rng.permutation(nb).astype(np.int32)
    dm = rng.integers(-16384, 16385, size=nb).astype(np.int32)
    dm[rng.choice(nb, size=max(1, nb // 8), replace=False)] = 0
    odt = TORCH_OF[out_dtype]
    out_k = canary_fill(torch.empty((L, nb, tb, H, 128), dtype=odt, device=DEV))
    out_v = canary_fill(torch.empty_like(out_k))
    tab = torch.from_numpy(table).to(DEV)
    dmt = torch.from_numpy(dm).to(DEV)
    order = hkv.page_visit_order(tab, nb)
    staging = hkv.alloc_staging(nb, fmt, tb, H, device=DEV)
    for b in staging:
        b.fill_(0xEE)
    main = torch.cuda.current_stream()
    fetch_stream = torch.cuda.Stream()
    copy_stream = torch.cuda.Stream() if separate_streams else fetch_stream
    compute = torch.cuda.Stream()
    ready = [torch.cuda.Event() for _ in range(L)]
    snap_k = torch.empty_like(out_k)
    snap_v = torch.empty_like(out_v)
    x = torch.randn((256, 1024), device=DEV)
    w = torch.randn((1024, 1024), device=DEV)
    start = torch.cuda.Event()
    start.record(main)
    fetch_stream.wait_event(start)
    compute.wait_event(start)
    torch.cuda.synchronize()
    hkv.fetch_staged(host_rec, fmt, tab, dmt, base, pairs, out_k, out_v, staging,
                     visit_order=order, copy_stream=copy_stream, fetch_stream=fetch_stream,
                     layer_ready=ready)
    with torch.cuda.stream(compute):
        for l in range(L):
            compute.wait_event(ready[l])          # layer l's pages are in place
            snap_k[l].copy_(out_k[l])
            snap_v[l].copy_(out_v[l])
            x = torch.tanh(x @ w * 0.03)          # the suffix compute of layer l
    torch.cuda.synchronize()
    assert torch.equal(snap_k.view(torch.uint8), out_k.view(torch.uint8)), \
        "the compute stream saw a layer before its fetch finished"
    assert torch.equal(snap_v.view(torch.uint8), out_v.view(torch.uint8))
    # every layer against the oracle
    kr, vd = O.fetch_exact(ref, fmt, tb, H, dm, base, pairs)
    kd, _ = O.dequant_records(ref, fmt, tb, H)
    kg = host_f64(out_k)[:, table]
    vg = host_f64(out_v)[:, table]
    check_values_exact(vg, O.round_output(vd, out_dtype), "staged V")
    zero = dm == 0
    check_values_exact(kg[:, zero], O.round_output(kd[:, zero], out_dtype), "staged K (dm = 0)")
    check_keys(kg[:, ~zero], kr[:, ~zero], kd[:, ~zero], out_dtype, "staged K")
    # the same as a fetch from device-resident records
    dev_rec = host_rec.to(DEV)
    ok2 = torch.empty_like(out_k)
    ov2 = torch.empty_like(out_v)
    hkv.fetch_dequant_rope_shift(dev_rec, fmt, tab, dmt, base, pairs, ok2, ov2,
                                 visit_order=order)
    torch.cuda.synchronize()
    assert torch.equal(ok2.view(torch.uint8), out_k.view(torch.uint8))
    assert torch.equal(ov2.view(torch.uint8), out_v.view(torch.uint8))


def test_staged_fetch_llama_like_8_layers():
    """FP8, bf16 pages, split-halves pairs, base 500000: 8 layers of 32
    blocks of 64 tokens x 8 heads, copies and fetches on separate streams
    (each staging buffer filled four times)."""
    print("[staged] 8 layers fp8 -> bf16", flush=True)
    _run(8, 32, 64, 8, "fp8", "bf16", "bf16", "half_split", 500000.0, seed=201,
         separate_streams=True)


def test_staged_fetch_int4_odd_layers():
    """INT4, fp16 pages, interleaved pairs, an odd layer count (9) and a
    ragged block (16 tokens x 3 heads)."""
    print("[staged] 9 layers int4 -> f16", flush=True)
    _run(9, 20, 16, 3, "int4", "f16", "f16", "interleaved", 10000.0, seed=202,
         separate_streams=True)


def test_staged_fetch_one_stream():
    """Copies and fetches on one stream: the same pages, no overlap."""
    print("[staged] one stream", flush=True)
    _run(3, 16, 16, 8, "fp8", "f32", "f32", "interleaved", 10000.0, seed=203,
         separate_streams=False)
