"""Seeded synthetic workloads for the KV codec: shapes, values, positions,
per-block position deltas and block tables.

This module holds no arithmetic of the method (no quantization, no RoPE, no
CRC).  It only draws random inputs, so the HIP path and the CPU oracle can be
fed identical data.

Workload shapes come from the model shapes the pages name: an 80-layer,
8-KV-head Llama-3-70B-shaped cache of 64k tokens (HyperCache post, Core
Design, layer-wise transfer paragraph) and a 36-layer, 8-KV-head Qwen3-8B
cache of 32k tokens in fp16 (KV-handoff module, section 1).  Values are
standard normal.

Post-RoPE keys: a rotation maps a pair of independent standard normals to a
pair of independent standard normals, so for the large workloads the cached
post-RoPE keys are drawn directly as N(0, 1).  The tiny workload instead draws
pre-RoPE keys, and the test that uses it applies RoPE at the cached positions
itself.
"""

from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

HEAD_DIM = 128


@dataclasses.dataclass(frozen=True)
class KVWorkload:
    name: str
    n_layers: int
    n_kv_heads: int
    n_tokens: int
    block_tokens: int
    src_dtype: str              # "f32" | "f16" | "bf16"
    out_dtype: str
    rope_base: float
    pairs: str                  # "interleaved" | "half_split"
    formats: tuple              # ("fp8",) / ("int4",) / ("fp8", "int4")
    delta_kind: str             # "const" | "uniform" | "reorder"
    delta_value: int = 0        # const delta, or bound of the uniform draw
    permute_pages: bool = True
    outlier_frac: float = 0.0   # fraction of (head, dim) channels scaled
    outlier_gain: float = 1.0
    seed: int = 0
    head_dim: int = HEAD_DIM

    @property
    def n_blocks(self) -> int:
        return -(-self.n_tokens // self.block_tokens)

    @property
    def n_vectors(self) -> int:
        """Head vectors per K or V tensor over all layers."""
        return self.n_layers * self.n_tokens * self.n_kv_heads


# The five workloads.  Readings where the workload descriptions are silent:
# pair convention and base for the 4-layer and INT4 cases follow the
# KV-handoff module's listing (interleaved, 10000); the Llama-shaped case uses
# the split-halves convention; INT4 blocks are 64 tokens.
TINY = KVWorkload(
    name="tiny_1L_8H_4x16_fp32", n_layers=1, n_kv_heads=8, n_tokens=64,
    block_tokens=16, src_dtype="f32", out_dtype="f32", rope_base=10000.0,
    pairs="interleaved", formats=("fp8",), delta_kind="const",
    delta_value=7168, permute_pages=False)

GQA_REORDER = KVWorkload(
    name="gqa_reorder_4L_8H_1344tok_fp32", n_layers=4, n_kv_heads=8,
    n_tokens=1344, block_tokens=16, src_dtype="f32", out_dtype="f32",
    rope_base=10000.0, pairs="interleaved", formats=("fp8", "int4"),
    delta_kind="reorder", permute_pages=False)

QWEN3_8B = KVWorkload(
    name="qwen3_8b_36L_8H_32768tok_fp16", n_layers=36, n_kv_heads=8,
    n_tokens=32768, block_tokens=64, src_dtype="f16", out_dtype="f16",
    rope_base=1e6, pairs="half_split", formats=("fp8",),
    delta_kind="uniform", delta_value=16384)

LLAMA3_70B = KVWorkload(
    name="llama3_70b_80L_8H_65536tok_bf16", n_layers=80, n_kv_heads=8,
    n_tokens=65536, block_tokens=64, src_dtype="bf16", out_dtype="bf16",
    rope_base=500000.0, pairs="half_split", formats=("fp8",),
    delta_kind="const", delta_value=8192)

# One GPU's share of the Llama-3-70B-shaped cache under tensor parallelism
# over its 8 KV heads (TP = 8): one head per GPU, everything else the same.
LLAMA3_70B_TP8 = KVWorkload(
    name="llama3_70b_tp8_shard_80L_1H_65536tok_bf16", n_layers=80, n_kv_heads=1,
    n_tokens=65536, block_tokens=64, src_dtype="bf16", out_dtype="bf16",
    rope_base=500000.0, pairs="half_split", formats=("fp8",),
    delta_kind="const", delta_value=8192)

INT4_L3 = KVWorkload(
    name="int4_l3_32L_8H_16384tok_fp16_outliers", n_layers=32, n_kv_heads=8,
    n_tokens=16384, block_tokens=64, src_dtype="f16", out_dtype="f16",
    rope_base=10000.0, pairs="interleaved", formats=("int4",),
    delta_kind="uniform", delta_value=4096, outlier_frac=0.01,
    outlier_gain=20.0)

ALL = (TINY, GQA_REORDER, QWEN3_8B, LLAMA3_70B, LLAMA3_70B_TP8, INT4_L3)

# GQA reorder chunks (tokens): cached order [Sys, DocA, DocB, Q], reused as
# [Sys, DocB, DocA, Q] (the HyperCache post's Part A experiment order).
REORDER_CHUNKS = (("Sys", 256), ("DocB", 512), ("DocA", 512), ("Q", 64))
REORDER_CACHED_ORDER = ("Sys", "DocA", "DocB", "Q")


def _seed_words(*parts) -> list:
    return [int(p) & 0xFFFFFFFF for p in parts]


def _rng(w: KVWorkload, *parts) -> np.random.Generator:
    return np.random.default_rng(_seed_words(w.seed, *parts))


# ---------------------------------------------------------------------------
# Values
# ---------------------------------------------------------------------------

def tiny_pre_rope_kv():
    """The tiny workload's pre-RoPE K then V, float32 [64, 8, 128], both from
    one generator seeded with 0."""
    g = np.random.default_rng(0)
    k = g.standard_normal((64, 8, HEAD_DIM)).astype(np.float32)
    v = g.standard_normal((64, 8, HEAD_DIM)).astype(np.float32)
    return k, v


def tiny_positions():
    """Cached positions 1024 + t of the tiny workload."""
    return 1024 + np.arange(64, dtype=np.int64)


def outlier_channels(w: KVWorkload, layer: int) -> np.ndarray:
    """Flat (head * head_dim + dim) indices of the outlier channels of a layer."""
    n_ch = w.n_kv_heads * w.head_dim
    n_out = int(round(w.outlier_frac * n_ch))
    if n_out == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(w, layer, 99).choice(n_ch, size=n_out, replace=False))


def host_layer_values(w: KVWorkload, layer: int, kv: int) -> np.ndarray:
    """One layer's K (kv=0) or V (kv=1) as float32 [T, H, 128] on the host,
    drawn from the (seed, layer, kv) substream; outlier channels scaled."""
    x = _rng(w, layer, kv).standard_normal((w.n_tokens, w.n_kv_heads, w.head_dim),
                                           dtype=np.float32)
    ch = outlier_channels(w, layer)
    if ch.size:
        flat = x.reshape(w.n_tokens, -1)
        flat[:, ch] *= np.float32(w.outlier_gain)
    return x


def device_seed(w: KVWorkload, layer: int, kv: int) -> int:
    h = hashlib.sha256(f"{w.name}:{w.seed}:{layer}:{kv}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def device_layer_values(w: KVWorkload, layer: int, kv: int, out, *, generator=None):
    """Fill `out` (a torch tensor viewable as [T, H, 128] on a GPU) with one
    layer's K or V drawn on the device, outlier channels scaled."""
    import torch
    g = generator if generator is not None else torch.Generator(device=out.device)
    g.manual_seed(device_seed(w, layer, kv))
    view = out.view(w.n_tokens, w.n_kv_heads * w.head_dim)
    view.normal_(0.0, 1.0, generator=g)
    ch = outlier_channels(w, layer)
    if ch.size:
        idx = torch.from_numpy(ch).to(out.device)
        view[:, idx] *= w.outlier_gain
    return out


# ---------------------------------------------------------------------------
# Positions, deltas and block tables
# ---------------------------------------------------------------------------

def delta_m(w: KVWorkload) -> np.ndarray:
    """Per-block position delta m_new - m_old (int32 [n_blocks])."""
    if w.delta_kind == "const":
        return np.full(w.n_blocks, w.delta_value, dtype=np.int32)
    if w.delta_kind == "uniform":
        b = w.delta_value
        return _rng(w, 7).integers(-b, b + 1, size=w.n_blocks).astype(np.int32)
    if w.delta_kind == "reorder":
        return reorder_plan(w)[1]
    raise ValueError(w.delta_kind)


def block_positions(w: KVWorkload):
    """(m_old, m_new) int32 [n_blocks]: the cached and the reused position of
    each logical block's first token, with m_new - m_old = delta_m(w).  Cached
    positions are the blocks' own token offsets (the reorder workload: their
    offsets in the cached order), raised by a common base so that no reused
    position is negative."""
    dm = delta_m(w).astype(np.int64)
    if w.delta_kind == "reorder":
        m_old = reorder_plan(w)[0].astype(np.int64) * w.block_tokens
    else:
        m_old = np.arange(w.n_blocks, dtype=np.int64) * w.block_tokens
    m_old += max(0, int(-(m_old + dm).min()))
    return m_old.astype(np.int32), (m_old + dm).astype(np.int32)


def reorder_plan(w: KVWorkload):
    """GQA reorder: for each block of the reused order, the block index it had
    in the cached order and its delta.  Returns (old_block[n_blocks],
    delta[n_blocks])."""
    tb = w.block_tokens
    sizes = dict(REORDER_CHUNKS)
    old_start, pos = {}, 0
    for name in REORDER_CACHED_ORDER:
        old_start[name] = pos
        pos += sizes[name]
    old_block, delta, new_pos = [], [], 0
    for name, n in REORDER_CHUNKS:
        for j in range(0, n, tb):
            old_block.append((old_start[name] + j) // tb)
            delta.append(new_pos + j - (old_start[name] + j))
        new_pos += n
    return np.asarray(old_block, dtype=np.int32), np.asarray(delta, dtype=np.int32)


def put_table(w: KVWorkload) -> np.ndarray:
    """Logical block -> source page for the put (int32 [n_blocks])."""
    if w.delta_kind == "reorder":
        return reorder_plan(w)[0]
    if not w.permute_pages:
        return np.arange(w.n_blocks, dtype=np.int32)
    return _rng(w, 5).permutation(w.n_blocks).astype(np.int32)


def fetch_table(w: KVWorkload) -> np.ndarray:
    """Logical block -> destination page for the fetch (int32 [n_blocks])."""
    if not w.permute_pages:
        return np.arange(w.n_blocks, dtype=np.int32)
    return _rng(w, 6).permutation(w.n_blocks).astype(np.int32)


def pages_from_tokens(x: np.ndarray, w: KVWorkload, table: np.ndarray) -> np.ndarray:
    """Place token-ordered values x[T, H, d] into pages [P, T_b, H, d] so that
    logical block b sits in page table[b] (pages not named stay zero)."""
    tb = w.block_tokens
    nb = w.n_blocks
    pad = nb * tb - x.shape[0]
    if pad:
        x = np.concatenate([x, np.zeros((pad,) + x.shape[1:], x.dtype)])
    blocks = x.reshape(nb, tb, *x.shape[1:])
    pages = np.zeros((int(table.max()) + 1 if table.size else 0,) + blocks.shape[1:], x.dtype)
    pages[table] = blocks
    return pages


# ---------------------------------------------------------------------------
# Layer-0 hidden states for the recompute selection
# ---------------------------------------------------------------------------
# A reused prefix is a list of chunks; the reorder moves every chunk after
# the leading system chunk.  The cached hidden states are N(0, 1).  The fresh
# ones equal them exactly on the leading chunk (same tokens at the same
# positions after the same predecessors) and elsewhere add N(0, sigma_t^2)
# noise, sigma_t = 0.05 * (1 + 4 exp(-j / 64)) * exp(0.5 z_t), j the token's
# offset in its chunk and z_t ~ N(0, 1): drift is largest right after a chunk
# boundary and log-normally spread, with a block of exact zeros (ties).

@dataclasses.dataclass(frozen=True)
class DriftWorkload:
    name: str
    lead_tokens: int            # the unmoved leading chunk
    chunk_tokens: int           # every later chunk
    n_chunks: int               # later chunks
    d_model: int
    dtype: str                  # "f32" | "f16" | "bf16"
    percent: int = 15
    seed: int = 0

    @property
    def n_tokens(self) -> int:
        return self.lead_tokens + self.n_chunks * self.chunk_tokens


# The GQA reorder's reused prefix [Sys 256, DocB 512, DocA 512] with a
# 32-query-head x 128 model width; Qwen3-8B (4096 wide, fp16) and
# Llama-3-70B (8192 wide, bf16) prefixes of 32k and 64k tokens.
DRIFT_GQA = DriftWorkload(name="drift_gqa_1280tok_4096_fp32", lead_tokens=256,
                          chunk_tokens=512, n_chunks=2, d_model=4096, dtype="f32")
DRIFT_QWEN3_8B = DriftWorkload(name="drift_qwen3_8b_32768tok_4096_fp16", lead_tokens=1024,
                               chunk_tokens=1024, n_chunks=31, d_model=4096, dtype="f16")
DRIFT_LLAMA3_70B = DriftWorkload(name="drift_llama3_70b_65536tok_8192_bf16", lead_tokens=2048,
                                 chunk_tokens=2048, n_chunks=31, d_model=8192, dtype="bf16")
DRIFT_ALL = (DRIFT_GQA, DRIFT_QWEN3_8B, DRIFT_LLAMA3_70B)


def drift_sigma(w: DriftWorkload) -> np.ndarray:
    """Per-token noise scale sigma_t (float32 [n_tokens]); 0 on the lead chunk."""
    z = np.random.default_rng(_seed_words(w.seed, 401, w.n_tokens)).standard_normal(
        w.n_tokens)
    j = (np.arange(w.n_tokens) - w.lead_tokens) % w.chunk_tokens
    s = 0.05 * (1.0 + 4.0 * np.exp(-j / 64.0)) * np.exp(0.5 * z)
    s[:w.lead_tokens] = 0.0
    return s.astype(np.float32)


def _round_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> the workload dtype, as float32 values (bf16 by RNE on the
    bit pattern)."""
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float32)
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def host_hidden_states(w: DriftWorkload):
    """(cached, fresh) float32 [n_tokens, d_model] holding values of the
    workload dtype, on the host."""
    g = np.random.default_rng(_seed_words(w.seed, 402, w.n_tokens))
    cached = _round_dtype(g.standard_normal((w.n_tokens, w.d_model), dtype=np.float32), w.dtype)
    noise = g.standard_normal((w.n_tokens, w.d_model), dtype=np.float32)
    fresh = _round_dtype(cached + drift_sigma(w)[:, None] * noise, w.dtype)
    return cached, fresh


def device_hidden_states(w: DriftWorkload, device, rows_per_step: int = 4096):
    """(cached, fresh) torch tensors [n_tokens, d_model] of the workload dtype
    drawn on `device`, row slab by row slab."""
    import torch
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
    cached = torch.empty((w.n_tokens, w.d_model), dtype=dt, device=device)
    fresh = torch.empty_like(cached)
    sigma = torch.from_numpy(drift_sigma(w)).to(device)
    g = torch.Generator(device=device)
    h = hashlib.sha256(f"{w.name}:{w.seed}:hidden".encode()).digest()
    g.manual_seed(int.from_bytes(h[:8], "little") & ((1 << 63) - 1))
    tmp = torch.empty((rows_per_step, w.d_model), dtype=torch.float32, device=device)
    for r0 in range(0, w.n_tokens, rows_per_step):
        r1 = min(w.n_tokens, r0 + rows_per_step)
        t = tmp[:r1 - r0]
        t.normal_(0.0, 1.0, generator=g)
        c = t.to(dt)
        cached[r0:r1] = c
        t.normal_(0.0, 1.0, generator=g)
        fresh[r0:r1] = (c.float() + sigma[r0:r1, None] * t).to(dt)
    return cached, fresh
