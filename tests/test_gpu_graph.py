"""The C ABI under HIP graph capture: put, CRC, page order, per-layer fetch,
per-token fetch, drift, top-k selection, the fused INT4 put + CRC and the
record frames (headers, verification) recorded once into a graph
(torch.cuda.CUDAGraph) and replayed.  The calls allocate nothing and do not
synchronize, so they can be captured; every replay must reproduce the eager
results bit for bit.  Between replays the outputs are scribbled over and other
eager work runs, and each replay is checked on its own."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from parity_util import TORCH_OF
from quantization_rope_reuse_amd import hkv
from quantization_rope_reuse_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_graph_capture_and_replay():
    w = W.GQA_REORDER
    L, nb, tb, H = w.n_layers, w.n_blocks, w.block_tokens, w.n_kv_heads
    print(f"[graph] {w.name}", flush=True)
    table = W.put_table(w)
    k = np.stack([W.pages_from_tokens(W.host_layer_values(w, l, 0), w, table) for l in range(L)])
    v = np.stack([W.pages_from_tokens(W.host_layer_values(w, l, 1), w, table) for l in range(L)])
    kp = torch.from_numpy(k).to(DEV, torch.bfloat16)
    vp = torch.from_numpy(v).to(DEV, torch.bfloat16)
    put_tab = torch.from_numpy(table).to(DEV)
    ftab = torch.from_numpy(W.fetch_table(w)).to(DEV)
    dm = torch.from_numpy(W.delta_m(w)).to(DEV)
    dm_tok = (dm.view(nb, 1) + torch.arange(tb, device=DEV, dtype=torch.int32) * 3).contiguous()
    dw = W.DRIFT_GQA
    hc, hf = W.host_hidden_states(dw)
    hc = torch.from_numpy(hc).to(DEV)
    hf = torch.from_numpy(hf).to(DEV)
    k_sel = O.recompute_count(dw.n_tokens)

    # static buffers, allocated before capture
    rec = hkv.alloc_records(L, nb, "fp8", tb, H, device=DEV)
    crc = torch.empty((L, nb), dtype=torch.int32, device=DEV)
    rec4 = hkv.alloc_records(L, nb, "int4", tb, H, device=DEV)      # fused put + CRC
    crc4 = torch.empty((L, nb), dtype=torch.int32, device=DEV)
    ws4 = torch.empty(hkv.quant_crc_workspace_bytes("int4", L, nb, tb, H), dtype=torch.uint8,
                      device=DEV)
    order = torch.empty(nb, dtype=torch.int32, device=DEV)
    ok = torch.empty((L, nb, tb, H, 128), dtype=torch.bfloat16, device=DEV)
    ov = torch.empty_like(ok)
    tk = torch.empty_like(ok)
    tv = torch.empty_like(ok)
    drift = torch.empty(dw.n_tokens, dtype=torch.float32, device=DEV)
    sel = torch.empty(k_sel, dtype=torch.int32, device=DEV)
    ws = torch.empty(hkv.select_workspace_bytes(dw.n_tokens), dtype=torch.uint8, device=DEV)
    fr = hkv.alloc_frames(L, nb, "fp8", tb, H, device=DEV)          # record frames
    fcrc = torch.empty((L, nb), dtype=torch.int32, device=DEV)
    fflags = torch.empty((L, nb), dtype=torch.int32, device=DEV)
    m_old = torch.from_numpy(W.block_positions(w)[0]).to(DEV)
    outs = (rec, crc, order, ok, ov, tk, tv, drift, sel, rec4, crc4, fr, fcrc, fflags)

    def step(stream=None):
        hkv.quant_fp8(kp, vp, put_tab, rec, stream=stream)
        hkv.crc32_blocks(rec, "fp8", tb, H, out=crc, stream=stream)
        hkv.page_visit_order(ftab, nb, out=order, stream=stream)
        for l in range(L):
            hkv.fetch_dequant_rope_shift(rec[l:l + 1], "fp8", ftab, dm, w.rope_base, w.pairs,
                                         ok[l:l + 1], ov[l:l + 1], visit_order=order,
                                         stream=stream)
        hkv.fetch_dequant_rope_shift_tokens(rec, "fp8", ftab, dm_tok, w.rope_base, w.pairs,
                                            tk, tv, stream=stream)
        hkv.token_drift(hc, hf, out=drift, stream=stream)
        hkv.select_top_tokens(drift, k_sel, out=sel, workspace=ws, stream=stream)
        hkv.quant_crc("int4", kp, vp, put_tab, rec4, crc_out=crc4, workspace=ws4, stream=stream)
        hkv.quant_fp8(kp, vp, put_tab, hkv.frame_records(fr), stream=stream)
        hkv.crc32_blocks(hkv.frame_records(fr), "fp8", tb, H, out=fcrc, stream=stream)
        hkv.frame_headers(fr, "fp8", tb, H, fcrc, m_old, stream=stream)
        hkv.frame_verify(fr, "fp8", tb, H, out=fflags, stream=stream)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]

    g = torch.cuda.CUDAGraph()
    for t in outs:
        t.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()                         # the current stream is the capture stream
    torch.cuda.synchronize()

    for replay in range(3):
        for t in outs:                 # scribble over every output, eagerly
            t.view(torch.uint8).fill_(0x5A + replay)
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        del junk
        for name, got, want in zip(("records", "crc", "order", "fetch K", "fetch V",
                                    "per-token K", "per-token V", "drift", "selection",
                                    "fused INT4 records", "fused INT4 CRC", "frames",
                                    "frame CRCs", "frame flags"),
                                   outs, eager):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), \
                f"replay {replay}: {name} differs from the eager run"
    # and the eager run itself against the oracle's selection on its drift
    assert np.array_equal(eager[8].cpu().numpy(), O.select_top_tokens(eager[7].cpu().numpy(),
                                                                     k_sel))
    # and the fused INT4 CRCs against the oracle's CRC of the records written
    got = eager[10].cpu().numpy().view(np.uint32)
    assert np.array_equal(got, O.crc32_records(eager[9].cpu().numpy()))
    # and the frames: every one intact, the same bytes as the oracle's frames
    assert not eager[13].cpu().numpy().any()
    want = O.make_frames(eager[0].cpu().numpy(), "fp8", tb, H, W.block_positions(w)[0])
    got_fr = eager[11].cpu().numpy()
    assert np.array_equal(got_fr[:, :, :want.shape[2]], want)
