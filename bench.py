"""Benchmark of the KV codec hot path on one MI355X.

Workload: a Llama-3-70B-shaped KV cache, 80 layers x 8 KV heads x 128 dims x
65,536 tokens in bf16 (21.5 GB), blocks of 64 tokens (1,024 pages per layer),
RoPE base 500000 with split-halves pairs, every block re-used 8,192 positions
later.  Synthetic standard-normal values drawn on the GPU.

One step is one pass of the whole hot path over that cache:
  1+2. put and CRC  FP8 E4M3 quantization of all 80 layers, gathered through a
            permuted block table into per-(layer, block) records (10.9 GB),
            with the CRC-32 of every record computed in the same pass
            (hkv_quant_fp8_crc: one put launch + a small merge launch);
  3. fetch  layer by layer on a side stream (80 launches): dequantize, shift
            keys by +8192, scatter into a second paged bf16 buffer through
            another permuted table, visiting blocks in destination-page order
            (computed once per step by the library's order kernel).
Inputs are resident in HBM before timing starts.

Reported (one JSON line on stdout):
  value        the metric: fetch GB/s = algorithmic fetch bytes of the 80
               layers / the fetch phase's time in the timed steps (HIP events
               on the fetch stream around its 80 launches)
  ms_per_step  the whole step (put + CRC + 80 fetches); `step` gives its rate
  roofline     the fetch kernel (the dominant one): algorithmic bytes per
               launch / mean launch time from the same HIP events, against
               8 TB/s HBM peak; also the mean launch time of the committed
               rocprofv3 kernel trace and the fraction it gives, while the
               fetch sources match the ones profiled; `traffic` = HBM bytes
               per launch from the committed rocprofv3 counters, likewise
  fetch        fetch GB/s, fraction of peak, tokens/s
  put_crc      the fused put + CRC phase; put, crc32: the same work as two
               separate passes, timed outside the step
  ceiling      a plain streaming kernel with the fetch's 1:2 byte mix, and the
               fetch as a fraction of it
  overlap      the layer-wise pipeline: records of all 80 layers in pinned
               host memory, copied layer by layer into two staging buffers
               and fetched from there (hkv_fetch_staged) while a compute
               stream runs a synthetic suffix GEMM per layer gated on each
               layer's fetch; exposed transfer + fetch time and the hidden
               fraction
  cpu_baseline the CPU oracle on a bounded sample of the same workload

Algorithmic bytes (what each step of the method covers):
  put    per vector 128 * 2 (bf16 read) + 128 + 2 (codes and scale written),
         plus the 4-byte table entry per (layer, block);
  CRC    per record its bytes plus 4 written (counted as the bytes the CRC
         covers; in the fused pass they come from LDS, not a second read);
  fetch  per vector 128 + 2 read + 128 * 2 written, plus the 4-byte table
         entry and 4-byte delta per (layer, block).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "KV fetch GB/s (fp8 dequant+RoPE shift+page scatter), % of HBM peak"


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--cpu-seconds", type=float, default=20.0,
                   help="approximate budget of the CPU-oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--layers", type=int, default=None,
                   help="override the layer count (profiling runs only)")
    p.add_argument("--overlap", action="store_true",
                   help="instead of the metric line, measure the layer-wise overlap of the "
                        "fetch with a synthetic suffix compute (bf16 GEMM per layer)")
    p.add_argument("--suffix-tokens", type=int, default=512,
                   help="suffix tokens of the synthetic per-layer compute (--overlap)")
    p.add_argument("--fetch-cus", type=int, nargs="*", default=[16, 32],
                   help="compute units given to the fetch stream in the CU-partitioned "
                        "overlap runs (--overlap)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a plain 1 GiB read + 1 GiB write elementwise kernel "
                        "(reference for scaling HBM byte counters)")
    return p.parse_args()


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "quantization_rope_reuse_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profiled_fetch_mean_ms():
    """Mean duration (ms) of the Llama-3-70B-shaped fetch launch in the
    committed rocprofv3 kernel trace, if it was taken on the current fetch
    sources; else None."""
    path = os.path.join(ROOT, "profiles", "llama3_70b_step_kernel_trace.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith((" ", "|", "(")):
                key, _, val = line.partition(":")
                fields[key.strip()] = val.strip()
    if fields.get("source_digest") != source_digest("fetch.hip", "hkv_device.h"):
        return None
    try:
        return float(fields["fetch_mean_us"]) / 1e3
    except (KeyError, ValueError):
        return None


def measured_traffic():
    """HBM bytes per fetch launch from the committed rocprofv3 counter
    summary, if it was taken on the current fetch sources; else None."""
    path = os.path.join(ROOT, "profiles", "fetch_llama3_70b_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith((" ", "|", "(")):
                key, _, val = line.partition(":")
                fields[key.strip()] = val.strip()
    if fields.get("source_digest") != source_digest("fetch.hip", "hkv_device.h"):
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {a.gpus} is not supported "
              "(the codec shards by layer, head or block with no exchange; see the design "
              "notes).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from quantization_rope_reuse_amd import hkv
    from quantization_rope_reuse_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    hkv.lib()                                   # fail loudly if not built
    dev = torch.device("cuda:0")
    w = W.LLAMA3_70B
    L = a.layers or w.n_layers
    T, H, tb, nb = w.n_tokens, w.n_kv_heads, w.block_tokens, w.n_blocks
    vecs_per_layer = 2 * T * H                  # K and V

    # ---- inputs resident in HBM -------------------------------------------
    t0 = time.perf_counter()
    src_k = torch.empty((L, nb, tb, H, 128), dtype=torch.bfloat16, device=dev)
    src_v = torch.empty_like(src_k)
    put_tab = torch.from_numpy(W.put_table(w)).to(dev)
    ftab = torch.from_numpy(W.fetch_table(w)).to(dev)
    dm = torch.from_numpy(W.delta_m(w)).to(dev)
    tmp = torch.empty((T, H, 128), dtype=torch.float32, device=dev)
    gen = torch.Generator(device=dev)
    for l in range(L):
        for kv, dst in ((0, src_k), (1, src_v)):
            W.device_layer_values(w, l, kv, tmp, generator=gen)
            dst[l].index_copy_(0, put_tab.long(), tmp.view(nb, tb, H, 128).to(torch.bfloat16))
    del tmp
    records = hkv.alloc_records(L, nb, "fp8", tb, H, device=dev)
    crc = torch.empty((L, nb), dtype=torch.int32, device=dev)
    crc_ws = torch.empty(hkv.quant_crc_workspace_bytes("fp8", L, nb, tb, H), dtype=torch.uint8,
                         device=dev)
    order = torch.empty(nb, dtype=torch.int32, device=dev)
    out_k = torch.empty_like(src_k)
    out_v = torch.empty_like(src_k)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0
    print(f"[bench] inputs ready: {L} layers, {2 * src_k.numel() * 2 / 1e9:.2f} GB bf16 source, "
          f"{records.numel() / 1e9:.2f} GB records ({setup_s:.1f} s)", file=sys.stderr, flush=True)

    main_stream = torch.cuda.current_stream(dev)
    side = torch.cuda.Stream(device=dev)
    rec_l = [records[l:l + 1] for l in range(L)]
    ok_l = [out_k[l:l + 1] for l in range(L)]
    ov_l = [out_v[l:l + 1] for l in range(L)]

    def step(ev=None):
        # ev: optional HIP events at the phase boundaries (none between the
        # per-layer fetch launches, which would add a gap between them)
        if ev is not None:
            ev[0].record(main_stream)
        # put and CRC in one pass (the put stages each workgroup's codes in
        # LDS and writes per-128-byte raw CRCs; a small kernel merges them)
        hkv.quant_crc("fp8", src_k, src_v, put_tab, records, crc_out=crc, workspace=crc_ws,
                      stream=main_stream)
        if ev is not None:
            ev[1].record(main_stream)
        ready = torch.cuda.Event()
        ready.record(main_stream)
        side.wait_event(ready)
        if ev is not None:
            ev[2].record(side)
        # blocks listed by destination page, shared by the 80 layer launches
        hkv.page_visit_order(ftab, nb, out=order, stream=side)
        for l in range(L):
            hkv.fetch_dequant_rope_shift(rec_l[l], "fp8", ftab, dm, w.rope_base, w.pairs,
                                         ok_l[l], ov_l[l], visit_order=order, stream=side)
        if ev is not None:
            ev[3].record(side)
        main_stream.wait_event(ev[3] if ev is not None else _record(side))

    def _record(stream):
        e = torch.cuda.Event()
        e.record(stream)
        return e

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / a.steps

    put_crc_ms = [e[0].elapsed_time(e[1]) for e in events]
    fetch_span_ms = [e[2].elapsed_time(e[3]) for e in events]
    fetch_ms = [f / L for f in fetch_span_ms]                  # mean per launch

    rb = hkv.record_bytes("fp8", tb, H)
    put_bytes = L * (vecs_per_layer * (256 + 130) + nb * 4)
    crc_bytes = L * nb * (rb + 4)
    fetch_launch_bytes = vecs_per_layer * (130 + 256) + nb * 8
    fetch_bytes = L * fetch_launch_bytes
    step_bytes = put_bytes + crc_bytes + fetch_bytes

    mean_fetch_ms = float(np.mean(fetch_ms))
    achieved = fetch_launch_bytes / (mean_fetch_ms * 1e-3) / 1e9
    fetch_gbps = fetch_bytes / (float(np.mean(fetch_span_ms)) * 1e-3) / 1e9
    tokens_per_s = T / (float(np.mean(fetch_span_ms)) * 1e-3)
    value = fetch_gbps                          # the metric: the fetch
    prof_ms = profiled_fetch_mean_ms()

    # quick integrity check of the last step: no page left unwritten
    if bool(torch.isnan(out_k).any()) or bool(torch.isnan(out_v).any()):
        raise RuntimeError("fetch produced NaN")

    # per-token deltas (the same +8192 for every token), 80 launches, timed once
    dm_tok = dm.view(nb, 1).expand(nb, tb).contiguous()

    def fetch_tokens_all():
        for l in range(L):
            hkv.fetch_dequant_rope_shift_tokens(rec_l[l], "fp8", ftab, dm_tok, w.rope_base,
                                                w.pairs, ok_l[l], ov_l[l], visit_order=order,
                                                stream=side)
    tok_ms = gpu_ms(side, fetch_tokens_all, 2)

    # the 80 per-layer fetch launches captured once in a HIP graph and replayed
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for l in range(L):
            hkv.fetch_dequant_rope_shift(rec_l[l], "fp8", ftab, dm, w.rope_base, w.pairs,
                                         ok_l[l], ov_l[l], visit_order=order)
    torch.cuda.synchronize()
    graph_ms = gpu_ms(torch.cuda.current_stream(dev), graph.replay, 3)
    del graph

    if a.overlap:
        print(json.dumps(overlap(a, w, L, hkv, rec_l, ok_l, ov_l, ftab, dm, order, side)),
              flush=True)
        return

    ceiling = stream_ceiling(dev, hkv, fetch_launch_bytes, fetch_gbps)
    separate = separate_put_crc(dev, hkv, L, nb, tb, H, src_k, src_v, put_tab, records, crc,
                                put_bytes, crc_bytes)
    put_ceiling = put_stream_ceiling(dev, hkv, separate["put"]["gbps"],
                                     put_bytes / (float(np.mean(put_crc_ms)) * 1e-3) / 1e9)
    staged = None
    if L == w.n_layers:
        staged = staged_overlap(dev, hkv, w, L, records, ftab, dm, order)
    frames = frames_leg(dev, hkv, W, w, L, src_k, src_v, put_tab)
    select = recompute_select(dev, hkv, W)
    others = other_workloads(dev, hkv, W)
    shard = tp8_shard(dev, hkv, W)

    if a.calibrate_copy:
        # torch.neg over 2**28 fp32 values: reads exactly 1 GiB, writes 1 GiB
        del src_k, src_v, out_k, out_v, records
        x = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        del x, y

    cpu = None
    if not a.no_cpu_baseline:
        cpu = cpu_baseline(w, records_bytes=rb, budget_s=a.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic N(0,1), generated on the GPU",
        "config": {
            "workload": "Llama-3-70B-shaped KV, one GPU: 80 layers x 8 KV heads x d128 x "
                        "65536 tokens bf16, blocks of 64, FP8 put + CRC32 in one pass + "
                        "layer-by-layer fetch on a side stream, dm=+8192, RoPE base 500000 "
                        "split-halves",
            "storage": "bf16 pages -> FP8 E4M3 records with fp16 scales -> bf16 pages "
                       "(arithmetic in fp32; per-block RoPE angles in fp64)",
            "layers": L, "tokens": T, "kv_heads": H, "head_dim": 128, "block_tokens": tb,
        },
        "step": {
            "ms": round(ms_per_step, 4),
            "bytes": step_bytes,
            "gbps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 2),
            "bytes_without_crc_reads": put_bytes + fetch_bytes,
            "gbps_without_crc_reads": round((put_bytes + fetch_bytes) / (ms_per_step * 1e-3)
                                            / 1e9, 2),
            "note": "put + CRC32 of every record + 80 fetches; the CRC covers 10.9 GB of "
                    "records that the fused pass reads from LDS, not HBM (left out in "
                    "*_without_crc_reads)",
        },
        "roofline": {
            "kernel": "fetch_kernel<fp8,bf16,half_split> (one layer per launch)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(),
            "alg_bytes_per_launch": fetch_launch_bytes,
            "mean_launch_ms": round(mean_fetch_ms, 5),
            "launch_ms_source": "HIP events on the fetch stream around the 80 per-layer "
                                "launches of each timed step (and the one visit-order "
                                "launch before them), divided by 80",
            "profile_mean_launch_ms": None if prof_ms is None else round(prof_ms, 5),
            "frac_at_profile_mean": None if prof_ms is None else round(
                fetch_launch_bytes / (prof_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "profile": "profiles/llama3_70b_step_kernel_trace.md (rocprofv3 per-dispatch "
                       "mean of the same launches; null when the fetch sources changed)",
        },
        "fetch": {
            "gbps": round(fetch_gbps, 1),
            "frac_of_peak": round(fetch_gbps / HBM_PEAK_GBPS, 4),
            "tokens_per_s": round(tokens_per_s, 0),
            "ms_80_layers": round(float(np.mean(fetch_span_ms)), 4),
            "ms_80_layers_median": round(float(np.median(fetch_span_ms)), 4),
            "ms_80_layers_min": round(float(np.min(fetch_span_ms)), 4),
            "gbps_at_median": round(fetch_bytes / (float(np.median(fetch_span_ms)) * 1e-3) / 1e9,
                                    1),
        },
        "ceiling": ceiling,
        "put_ceiling": put_ceiling,
        "fetch_per_token_delta": {
            "gbps": round(fetch_bytes / (tok_ms * 1e-3) / 1e9, 1),
            "ms_80_layers": round(tok_ms, 4),
            "note": "hkv_fetch_dequant_rope_shift_tokens, one delta per token",
        },
        "fetch_graph": {
            "ms_80_layers": round(graph_ms, 4),
            "gbps": round(fetch_bytes / (graph_ms * 1e-3) / 1e9, 1),
            "note": "the same 80 per-layer launches captured once in a HIP graph, replayed",
        },
        "put_crc": {"mean_ms": round(float(np.mean(put_crc_ms)), 4),
                    "median_ms": round(float(np.median(put_crc_ms)), 4),
                    "min_ms": round(float(np.min(put_crc_ms)), 4),
                    "gbps": round((put_bytes + crc_bytes) / (float(np.mean(put_crc_ms)) * 1e-3)
                                  / 1e9, 1),
                    "note": "hkv_quant_fp8_crc: put and CRC-32 in one pass (the step's "
                            "phase); CRC bytes counted as the record bytes it covers"},
        "put": separate["put"],
        "crc32": separate["crc32"],
        "other_workloads": others,
        "tp8_shard": shard,
        "overlap": staged,
        "frames": frames,
        "recompute_select": select,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def gpu_ms(stream, fn, reps):
    """Mean GPU time per call of fn() over `reps` back-to-back calls on
    `stream`, from HIP events.  One untimed call goes first, so the GPU is
    busy while the timed calls are enqueued and the host's own time per call
    stays outside the events (every leg timed this way runs far longer on
    the GPU than its call takes on the host)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    fn()
    ev[0].record(stream)
    for _ in range(reps):
        fn()
    ev[1].record(stream)
    stream.synchronize()
    return ev[0].elapsed_time(ev[1]) / reps


def stream_ceiling(dev, hkv, fetch_launch_bytes, fetch_gbps, nbuf=16, reps=64):
    """The fetch's byte mix with nothing else to do: hkv_stream_probe reads
    one fetch layer's worth of bytes (136 MB) and writes twice that, with the
    fetch's store pattern, rotating over 16 buffer pairs (more than the
    256 MB Infinity Cache).  HIP events on the current stream."""
    import torch
    n_read = 1040 * 1024 * 128          # 136,314,880 B: the codes and scales of one layer
    src = [torch.full((n_read,), 7, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
    dst = [torch.empty(2 * n_read, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
    s = torch.cuda.current_stream(dev)
    for i in range(2 * nbuf):
        hkv.stream_probe(src[i % nbuf], dst[i % nbuf], stream=s)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(s)
    for i in range(reps):
        hkv.stream_probe(src[i % nbuf], dst[i % nbuf], stream=s)
    ev[1].record(s)
    s.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    gbps = 3 * n_read / (ms * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"kernel": "hkv_stream_probe: 1 byte read for 2 written, 136 MB read per launch, "
                      "the fetch's non-temporal store pattern",
            "gbps": round(gbps, 1),
            "us_per_launch": round(ms * 1e3, 2),
            "fetch_frac_of_ceiling": round(fetch_gbps / gbps, 4)}


def put_stream_ceiling(dev, hkv, put_gbps, put_crc_put_gbps, nbuf=16, reps=64):
    """The put's byte mix with nothing else to do: hkv_stream_probe_put reads
    272 MB and writes 136 MB per launch (two source bytes per record byte)
    with the put's load and store pattern, rotating over 16 buffer pairs.
    HIP events on the current stream.  The put alone and the fused put + CRC
    pass (counted in put bytes only) are reported as fractions of it."""
    import torch
    n_write = 1040 * 1024 * 128
    src = [torch.full((2 * n_write,), 7, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
    dst = [torch.empty(n_write, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
    s = torch.cuda.current_stream(dev)
    for i in range(2 * nbuf):
        hkv.stream_probe_put(src[i % nbuf], dst[i % nbuf], stream=s)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(s)
    for i in range(reps):
        hkv.stream_probe_put(src[i % nbuf], dst[i % nbuf], stream=s)
    ev[1].record(s)
    s.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    gbps = 3 * n_write / (ms * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"kernel": "hkv_stream_probe_put: 2 bytes read for 1 written, 272 MB read per launch, "
                      "the put's load and non-temporal store pattern",
            "gbps": round(gbps, 1),
            "us_per_launch": round(ms * 1e3, 2),
            "put_frac_of_ceiling": round(put_gbps / gbps, 4),
            "put_crc_frac_of_ceiling": round(put_crc_put_gbps / gbps, 4)}


def separate_put_crc(dev, hkv, L, nb, tb, H, src_k, src_v, put_tab, records, crc, put_bytes,
                     crc_bytes, reps=5):
    """The put (hkv_quant_fp8) and the CRC (hkv_crc32_blocks) as two passes over
    the same cache, each timed with HIP events on the current stream; their
    CRCs must equal the fused pass's from the step."""
    import torch
    s = torch.cuda.current_stream(dev)
    crc2 = torch.empty_like(crc)
    pm = gpu_ms(s, lambda: hkv.quant_fp8(src_k, src_v, put_tab, records, stream=s), reps)
    cm = gpu_ms(s, lambda: hkv.crc32_blocks(records, "fp8", tb, H, out=crc2, stream=s), reps)
    if not torch.equal(crc, crc2):
        raise RuntimeError("the CRC kernel disagrees with the fused put + CRC")
    return {"put": {"mean_ms": round(pm, 4), "gbps": round(put_bytes / (pm * 1e-3) / 1e9, 1),
                    "note": "hkv_quant_fp8 alone"},
            "crc32": {"mean_ms": round(cm, 4), "gbps": round(crc_bytes / (cm * 1e-3) / 1e9, 1),
                      "note": "hkv_crc32_blocks alone (records read back)"}}


def other_workloads(dev, hkv, W, reps=10):
    """Put, put + CRC-32 in one pass, and fetch throughput on the Qwen3-8B-shaped
    (FP8, fp16 pages, random per-block deltas) and INT4 disk-tier (fp16 with
    outlier channels) caches, all layers in one call per operation.  Outside
    the step; HIP events."""
    import torch
    res = {}
    for w, fmt in ((W.QWEN3_8B, "fp8"), (W.INT4_L3, "int4")):
        L, nb, tb, H = w.n_layers, w.n_blocks, w.block_tokens, w.n_kv_heads
        dt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[w.src_dtype]
        src_k = torch.empty((L, nb, tb, H, 128), dtype=dt, device=dev)
        src_v = torch.empty_like(src_k)
        put_tab = torch.from_numpy(W.put_table(w)).to(dev)
        tmp = torch.empty((w.n_tokens, H, 128), dtype=torch.float32, device=dev)
        gen = torch.Generator(device=dev)
        for l in range(L):
            for kv, dst in ((0, src_k), (1, src_v)):
                W.device_layer_values(w, l, kv, tmp, generator=gen)
                dst[l].index_copy_(0, put_tab.long(), tmp.view(nb, tb, H, 128).to(dt))
        del tmp
        rec = hkv.alloc_records(L, nb, fmt, tb, H, device=dev)
        ftab = torch.from_numpy(W.fetch_table(w)).to(dev)
        dm = torch.from_numpy(W.delta_m(w)).to(dev)
        order = hkv.page_visit_order(ftab, nb)
        out_k = torch.empty_like(src_k)
        out_v = torch.empty_like(src_k)
        put = hkv.quant_fp8 if fmt == "fp8" else hkv.quant_int4
        s = torch.cuda.current_stream(dev)
        pms = gpu_ms(s, lambda: put(src_k, src_v, put_tab, rec, stream=s), reps)
        fms = gpu_ms(s, lambda: hkv.fetch_dequant_rope_shift(
            rec, fmt, ftab, dm, w.rope_base, w.pairs, out_k, out_v, visit_order=order,
            stream=s), reps)
        # the put with the CRC-32 of every record in one pass (the disk tier
        # writes its records with their CRCs)
        crc = torch.empty((L, nb), dtype=torch.int32, device=dev)
        ws = torch.empty(max(16, hkv.quant_crc_workspace_bytes(fmt, L, nb, tb, H)),
                         dtype=torch.uint8, device=dev)
        pcms = gpu_ms(s, lambda: hkv.quant_crc(fmt, src_k, src_v, put_tab, rec, crc_out=crc,
                                               workspace=ws, stream=s), reps)
        del crc, ws
        cb = 128 if fmt == "fp8" else 64
        vecs = 2 * L * w.n_tokens * H
        es = src_k.element_size()
        fetch_bytes = vecs * (cb + 2 + 128 * es) + L * nb * 8
        put_bytes = vecs * (128 * es + cb + 2) + L * nb * 4
        res[w.name] = {
            "format": fmt,
            "fetch_ms": round(fms, 4),
            "fetch_gbps": round(fetch_bytes / (fms * 1e-3) / 1e9, 1),
            "fetch_frac_of_peak": round(fetch_bytes / (fms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "fetch_tokens_per_s": round(w.n_tokens / (fms * 1e-3), 0),
            "put_ms": round(pms, 4),
            "put_gbps": round(put_bytes / (pms * 1e-3) / 1e9, 1),
            "put_crc_ms": round(pcms, 4),
            "put_crc_gbps_put_bytes": round(put_bytes / (pcms * 1e-3) / 1e9, 1),
        }
        del src_k, src_v, rec, out_k, out_v
        torch.cuda.empty_cache()
    return res


def tp8_shard(dev, hkv, W, reps=5):
    """One GPU's share of the Llama-3-70B-shaped cache under tensor
    parallelism over its 8 KV heads: one head, 131,072 vectors per layer
    (17.0 MB read and 33.6 MB written per layer fetch).  Put and CRC in one
    pass, then the 80 per-layer fetches on one stream, launched eagerly and
    replayed from a HIP graph.  Outside the step; HIP events."""
    import torch
    w = W.LLAMA3_70B_TP8
    L, nb, tb, H = w.n_layers, w.n_blocks, w.block_tokens, w.n_kv_heads
    src_k = torch.empty((L, nb, tb, H, 128), dtype=torch.bfloat16, device=dev)
    src_v = torch.empty_like(src_k)
    put_tab = torch.from_numpy(W.put_table(w)).to(dev)
    tmp = torch.empty((w.n_tokens, H, 128), dtype=torch.float32, device=dev)
    gen = torch.Generator(device=dev)
    for l in range(L):
        for kv, dst in ((0, src_k), (1, src_v)):
            W.device_layer_values(w, l, kv, tmp, generator=gen)
            dst[l].index_copy_(0, put_tab.long(), tmp.view(nb, tb, H, 128).to(torch.bfloat16))
    del tmp
    rec = hkv.alloc_records(L, nb, "fp8", tb, H, device=dev)
    crc = torch.empty((L, nb), dtype=torch.int32, device=dev)
    ws = torch.empty(hkv.quant_crc_workspace_bytes("fp8", L, nb, tb, H), dtype=torch.uint8,
                     device=dev)
    ftab = torch.from_numpy(W.fetch_table(w)).to(dev)
    dm = torch.from_numpy(W.delta_m(w)).to(dev)
    order = hkv.page_visit_order(ftab, nb)
    out_k = torch.empty_like(src_k)
    out_v = torch.empty_like(src_k)
    rec_l = [rec[l:l + 1] for l in range(L)]
    ok_l = [out_k[l:l + 1] for l in range(L)]
    ov_l = [out_v[l:l + 1] for l in range(L)]
    s = torch.cuda.current_stream(dev)

    def fetch_all():
        for l in range(L):
            hkv.fetch_dequant_rope_shift(rec_l[l], "fp8", ftab, dm, w.rope_base, w.pairs,
                                         ok_l[l], ov_l[l], visit_order=order, stream=s)

    pms = gpu_ms(s, lambda: hkv.quant_crc("fp8", src_k, src_v, put_tab, rec, crc_out=crc,
                                          workspace=ws, stream=s), reps)
    fms = gpu_ms(s, fetch_all, reps)
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for l in range(L):
            hkv.fetch_dequant_rope_shift(rec_l[l], "fp8", ftab, dm, w.rope_base, w.pairs,
                                         ok_l[l], ov_l[l], visit_order=order)
    torch.cuda.synchronize()
    gms = gpu_ms(torch.cuda.current_stream(dev), graph.replay, reps)
    del graph
    # the same 80 layers in one call (one launch): the kernel without the
    # per-launch ramp and drain
    oms = gpu_ms(s, lambda: hkv.fetch_dequant_rope_shift(
        rec, "fp8", ftab, dm, w.rope_base, w.pairs, out_k, out_v, visit_order=order,
        stream=s), reps)
    vecs_layer = 2 * w.n_tokens * H
    launch_bytes = vecs_layer * (130 + 256) + nb * 8
    put_bytes = L * (vecs_layer * (256 + 130) + nb * 4)
    crc_bytes = L * nb * (hkv.record_bytes("fp8", tb, H) + 4)
    res = {
        "workload": "Llama-3-70B-shaped cache, one KV head (one GPU of TP = 8): 80 layers x "
                    "65536 tokens x 1 head x d128 bf16, blocks of 64, dm=+8192",
        "fetch_bytes_per_layer": launch_bytes,
        "fetch_ms_80_layers": round(fms, 4),
        "fetch_us_per_layer": round(fms * 1e3 / L, 2),
        "fetch_gbps": round(L * launch_bytes / (fms * 1e-3) / 1e9, 1),
        "fetch_frac_of_peak": round(L * launch_bytes / (fms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "fetch_graph_ms_80_layers": round(gms, 4),
        "fetch_graph_gbps": round(L * launch_bytes / (gms * 1e-3) / 1e9, 1),
        "fetch_one_launch_ms_80_layers": round(oms, 4),
        "fetch_one_launch_gbps": round(L * launch_bytes / (oms * 1e-3) / 1e9, 1),
        "put_crc_ms": round(pms, 4),
        "put_crc_gbps": round((put_bytes + crc_bytes) / (pms * 1e-3) / 1e9, 1),
    }
    del src_k, src_v, rec, out_k, out_v, rec_l, ok_l, ov_l
    torch.cuda.empty_cache()
    return res


def staged_overlap(dev, hkv, w, L, records, ftab, dm, order, suffix_tokens=2048, reps=3):
    """The layer-wise pipeline of the HyperCache post (layer l+1 is brought
    into a staging buffer while layer l's suffix tokens are computed) with a
    real transfer: the FP8 records of all 80 layers sit in pinned host memory
    and hkv_fetch_staged copies them layer by layer (DMA, copy stream) into
    two device staging buffers and fetches each layer from there (fetch
    stream).  The suffix compute is a synthetic bf16 GEMM with one
    Llama-3-70B layer's weights ([S x 8192] @ [8192 x 106496], S suffix
    tokens) per layer on a compute stream; layer l's GEMM waits on layer l's
    ready event.  Timed with wall clock around each whole run (best of
    `reps`): the transfer + fetch alone, the compute alone, and both
    overlapped; exposed = overlapped - compute alone."""
    import torch
    nb, tb, H = w.n_blocks, w.block_tokens, w.n_kv_heads
    rb = records.shape[2]
    full = records.as_strided((L, nb, records.stride(1)), records.stride())
    t0 = time.perf_counter()
    host = torch.empty(full.shape, dtype=torch.uint8).pin_memory()
    host.copy_(full)
    host_rec = host[:, :, :rb]
    staging = hkv.alloc_staging(nb, "fp8", tb, H, device=dev)
    out_k = torch.empty((L, nb, tb, H, 128), dtype=torch.bfloat16, device=dev)
    out_v = torch.empty_like(out_k)
    x = torch.randn((suffix_tokens, 8192), dtype=torch.bfloat16, device=dev)
    wt = torch.randn((8192, 106496), dtype=torch.bfloat16, device=dev) * 0.01
    y = torch.empty((suffix_tokens, 106496), dtype=torch.bfloat16, device=dev)
    copy_s, fetch_s, comp_s = (torch.cuda.Stream(device=dev) for _ in range(3))
    ready = [torch.cuda.Event() for _ in range(L)]
    torch.cuda.synchronize()
    print(f"[bench] overlap leg: {host.numel() / 1e9:.2f} GB of records pinned in host memory "
          f"({time.perf_counter() - t0:.1f} s)", file=sys.stderr, flush=True)

    def staged():
        hkv.fetch_staged(host_rec, "fp8", ftab, dm, w.rope_base, w.pairs, out_k, out_v, staging,
                         visit_order=order, copy_stream=copy_s, fetch_stream=fetch_s,
                         layer_ready=ready)

    def compute(gated):
        with torch.cuda.stream(comp_s):
            for l in range(L):
                if gated:
                    comp_s.wait_event(ready[l])
                torch.matmul(x, wt, out=y)

    def timed(fn):
        best = None
        for _ in range(reps):
            torch.cuda.synchronize()
            t = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t) * 1e3
            best = dt if best is None else min(best, dt)
        return best

    staged()
    compute(False)
    tf = timed(staged)
    tc = timed(lambda: compute(False))
    to = timed(lambda: (staged(), compute(True)))
    # every layer's pages of the overlapped run against a fetch from device
    # memory (bitwise)
    ok2 = torch.empty_like(out_k[:1])
    ov2 = torch.empty_like(out_v[:1])
    for l in range(L):
        hkv.fetch_dequant_rope_shift(records[l:l + 1], "fp8", ftab, dm, w.rope_base, w.pairs,
                                     ok2, ov2, visit_order=order)
        if not (torch.equal(ok2[0].view(torch.uint8), out_k[l].view(torch.uint8))
                and torch.equal(ov2[0].view(torch.uint8), out_v[l].view(torch.uint8))):
            raise RuntimeError(f"the staged fetch disagrees with the fetch from device memory "
                               f"in layer {l}")
    extent = (nb - 1) * host_rec.stride(1) + rb
    exposed = to - tc
    res = {
        "workload": f"{L} layers of FP8 records ({L * extent / 1e9:.2f} GB) in pinned host "
                    f"memory -> 2 staging buffers -> bf16 pages; suffix compute "
                    f"[{suffix_tokens} x 8192] @ [8192 x 106496] bf16 per layer",
        "transfer_fetch_ms": round(tf, 3),
        "h2d_gbps": round(L * extent / (tf * 1e-3) / 1e9, 2),
        "compute_ms": round(tc, 3),
        "overlapped_ms": round(to, 3),
        "serial_ms": round(tf + tc, 3),
        "exposed_fetch_ms": round(exposed, 3),
        "hidden_fraction": round(min(1.0, max(0.0, 1.0 - exposed / tf)), 4),
    }
    del host, host_rec, staging, out_k, out_v, x, wt, y, ok2, ov2
    torch.cuda.empty_cache()
    return res


def frames_leg(dev, hkv, W, w, L, src_k, src_v, put_tab, reps=3):
    """The same cache as self-describing frames (64-byte header + record):
    put into the frames' records, CRC, header writing, and a full
    verification (CRC of every record again plus the header checks).
    Outside the step; HIP events on the current stream."""
    import numpy as np
    import torch
    nb, tb, H = w.n_blocks, w.block_tokens, w.n_kv_heads
    frames = hkv.alloc_frames(L, nb, "fp8", tb, H, device=dev)
    rec = hkv.frame_records(frames)
    crc = torch.empty((L, nb), dtype=torch.int32, device=dev)
    crc_ws = torch.empty(hkv.quant_crc_workspace_bytes("fp8", L, nb, tb, H), dtype=torch.uint8,
                         device=dev)
    flags = torch.empty((L, nb), dtype=torch.int32, device=dev)
    m_old = torch.from_numpy(W.block_positions(w)[0]).to(dev)
    s = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    hdr_ms, ver_ms = [], []
    for rep in range(reps + 1):
        ev[0].record(s)
        hkv.quant_fp8(src_k, src_v, put_tab, rec, stream=s)
        hkv.crc32_blocks(rec, "fp8", tb, H, out=crc, stream=s)
        ev[1].record(s)
        hkv.frame_headers(frames, "fp8", tb, H, crc, m_old, stream=s)
        ev[2].record(s)
        hkv.frame_verify(frames, "fp8", tb, H, out=flags, stream=s)
        ev[3].record(s)
        s.synchronize()
        if rep:
            hdr_ms.append(ev[1].elapsed_time(ev[2]))
            ver_ms.append(ev[2].elapsed_time(ev[3]))
    if bool(flags.any()):
        raise RuntimeError("frame verification flagged intact frames")
    rb = hkv.record_bytes("fp8", tb, H)
    verify_bytes = L * nb * (rb + 64 + 4)
    vms = float(np.mean(ver_ms))
    del frames, rec
    torch.cuda.empty_cache()
    return {
        "frames": L * nb,
        "frame_bytes": 64 + rb,
        "headers_ms": round(float(np.mean(hdr_ms)), 4),
        "verify_ms": round(vms, 4),
        "verify_gbps": round(verify_bytes / (vms * 1e-3) / 1e9, 1),
    }


def recompute_select(dev, hkv, W, reps=10):
    """The recompute selection on a Llama-3-70B-width prefix (65,536 tokens x
    8,192 bf16): per-token layer-0 drift, then the top 15%.  Outside the
    step; timed with HIP events on the current stream.  Algorithmic bytes of
    the drift: both rows read (2 * 8192 * 2 per token) plus the fp32 drift."""
    import torch
    w = W.DRIFT_LLAMA3_70B
    cached, fresh = W.device_hidden_states(w, dev)
    drift = torch.empty(w.n_tokens, dtype=torch.float32, device=dev)
    k = (w.n_tokens * w.percent) // 100
    sel = torch.empty(k, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream(dev)
    dms = gpu_ms(s, lambda: hkv.token_drift(cached, fresh, out=drift, stream=s), reps)
    sms = gpu_ms(s, lambda: hkv.select_top_tokens(drift, k, out=sel, stream=s), reps)
    es = cached.element_size()
    drift_bytes = w.n_tokens * (2 * w.d_model * es + 4)
    gbps = drift_bytes / (dms * 1e-3) / 1e9
    del cached, fresh
    torch.cuda.empty_cache()
    return {
        "workload": f"{w.n_tokens} tokens x {w.d_model} {w.dtype} layer-0 hidden states, "
                    f"top {w.percent}% (k={k})",
        "drift_ms": round(dms, 4),
        "drift_gbps": round(gbps, 1),
        "drift_frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "drift_alg_bytes": drift_bytes,
        "select_ms": round(sms, 4),
    }


def overlap(a, w, L, hkv, rec_l, ok_l, ov_l, ftab, dm, order, side):
    """Layer-wise overlap (the HyperCache post's layer-wise transfer
    paragraph): the fetch of layer l+1 runs on a side stream while the main
    stream runs layer l's suffix compute, which needs layer l's fetched KV.
    The suffix compute is a synthetic bf16 GEMM with the FLOPs of one
    Llama-3-70B layer over `suffix_tokens` tokens (2 * S * 70e9 / 80).
    Measured twice: with two ordinary streams (the GEMM may hold every CU),
    and with hkv_stream_pair_create's CU-partitioned streams."""
    import torch

    dev = rec_l[0].device
    S = a.suffix_tokens
    x = torch.randn((S, 8192), dtype=torch.bfloat16, device=dev)
    wt = torch.randn((8192, 106496), dtype=torch.bfloat16, device=dev) * 0.01
    y = torch.empty((S, 106496), dtype=torch.bfloat16, device=dev)

    def timed(fn, reps=3):
        best = None
        for _ in range(reps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) * 1e3
            best = dt if best is None else min(best, dt)
        return best

    def run(fetch_stream, compute_stream):
        def fetch(l):
            hkv.fetch_dequant_rope_shift(rec_l[l], "fp8", ftab, dm, w.rope_base, w.pairs,
                                         ok_l[l], ov_l[l], visit_order=order,
                                         stream=fetch_stream)

        def compute_only():
            with torch.cuda.stream(compute_stream):
                for _ in range(L):
                    torch.matmul(x, wt, out=y)

        def fetch_only():
            for l in range(L):
                fetch(l)

        def overlapped():
            done = [torch.cuda.Event() for _ in range(L)]
            start = torch.cuda.Event()
            start.record(torch.cuda.current_stream(dev))
            fetch_stream.wait_event(start)
            compute_stream.wait_event(start)
            for l in range(L):            # the fetch stream runs ahead, layer by layer
                fetch(l)
                done[l].record(fetch_stream)
            with torch.cuda.stream(compute_stream):
                for l in range(L):
                    compute_stream.wait_event(done[l])   # layer l needs its KV
                    torch.matmul(x, wt, out=y)

        timed(compute_only, 1)
        c, f, o = timed(compute_only), timed(fetch_only), timed(overlapped)
        return {"compute_only_ms": round(c, 3), "fetch_only_ms": round(f, 3),
                "overlapped_ms": round(o, 3), "exposed_fetch_ms": round(o - c, 3),
                "hidden_fraction_of_fetch": round(1.0 - max(0.0, o - c) / f, 4)}

    out = {"mode": "layer-wise overlap", "layers": L, "suffix_tokens": S,
           "gemm": f"[{S} x 8192] @ [8192 x 106496] bf16 per layer (torch.matmul)",
           "ordinary_streams": run(side, torch.cuda.Stream(device=dev))}
    for n in a.fetch_cus:
        pair = hkv.StreamPair(n, device=dev)
        try:
            out[f"cu_partition_{n}"] = run(pair.fetch, pair.compute)
        finally:
            pair.close()
    return out


def cpu_baseline(w, records_bytes, budget_s):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    put + CRC + fetch of the first n blocks of a layer, n sized from two short
    calibration runs so that the measured run takes about 0.8 * `budget_s`
    (whole layers are added when one layer is not enough).  Reported in GB/s
    of the same algorithmic bytes as the GPU figures."""
    import numpy as np

    import oracle as O
    from quantization_rope_reuse_amd import workloads as W

    T, H, tb, nb = w.n_tokens, w.n_kv_heads, w.block_tokens, w.n_blocks
    dm_all = W.delta_m(w)

    def run(layer, n):
        k_all = W.host_layer_values(w, layer, 0)
        v_all = W.host_layer_values(w, layer, 1)
        # the source dtype is bf16: round the drawn values first (input prep)
        kb = O.f32_to_bf16_value(k_all[: n * tb]).astype(np.float32).reshape(1, n, tb, H, 128)
        vb = O.f32_to_bf16_value(v_all[: n * tb]).astype(np.float32).reshape(1, n, tb, H, 128)
        table = np.arange(n)
        c0 = time.process_time()
        t0 = time.perf_counter()
        rec, _ = O.put(kb, vb, table, O.FMT_FP8)
        O.crc32_records(rec)
        ko = np.zeros((1, n, tb, H, 128))
        vo = np.zeros((1, n, tb, H, 128))
        O.fetch(rec, O.FMT_FP8, tb, H, table, dm_all[:n], w.rope_base, w.pairs, ko, vo, "bf16")
        return time.perf_counter() - t0, time.process_time() - c0

    # calibration: fixed and per-block time from two short runs
    t32, _ = run(0, 32)
    t128, _ = run(0, 128)
    per_block = max((t128 - t32) / 96, 1e-6)
    fixed = max(t32 - 32 * per_block, 0.0)
    n = min(nb, max(1, int((0.8 * budget_s - fixed) / per_block)))
    wall, cpu_t = run(0, n)                     # the measured sample
    blocks, layers = n, 1
    while n == nb and wall * (layers + 1) / layers < budget_s and layers < w.n_layers:
        wl, cl = run(layers, nb)
        wall, cpu_t, blocks, layers = wall + wl, cpu_t + cl, blocks + nb, layers + 1
    vecs = 2 * blocks * tb * H
    alg = (vecs * (256 + 130) + blocks * 4 + blocks * (records_bytes + 4)
           + vecs * (130 + 256) + blocks * 8)
    return {
        "value": round(alg / wall / 1e9, 5),
        "unit": "GB/s",
        "cores": max(1, int(round(cpu_t / wall))),
        "cores_available": len(os.sched_getaffinity(0)),
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": f"put + CRC32 + fetch of {blocks} blocks ({blocks * tb} tokens, {layers} "
                  f"layer(s)) of the same workload, numpy float64 oracle, {wall:.1f} s wall, "
                  f"{cpu_t:.1f} s CPU",
    }


if __name__ == "__main__":
    main()
