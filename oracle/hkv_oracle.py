"""CPU oracle for the KV-block codec and the relative RoPE shift.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library.

It is deliberately plain and slow: numpy in float64 plus integer bit
operations, whole-array steps in the order the pages describe, no blocking or
fusion.  Every floating-point value is carried in float64, where each rounding
step the method defines (fp32 quotient, fp16 scale, FP8/INT4 code, fp32 /
fp16 / bf16 output) is applied explicitly and exactly.

Sources (web pages; cited by title and section):

* "HyperCache – Distributed KV-cache quantization and relative RoPE reuse"
  (called "the HyperCache post" below).
    - Core Design, relative-RoPE paragraph and its SO(2) identity: a cached
      post-RoPE key reused at a new offset is rotated pair by pair by
      (m_new - m_old) * theta_i; values are not rotated.
    - Core Design, compression paragraph, and the Part B benchmark printout:
      FP8 (E4M3) wire records, INT4 grouped disk records with CRC32, their
      compression ratios and byte counts.
* "Модуль 13: KV-хэндофф: передача кеша между моделями и узлами" (LLM
  Inference Systems course; called "the KV-handoff module" below).
    - Section 1 formula for KV bytes.
    - The module13.py listing, functions rope_cache / apply_rope /
      strip_rope: the angle table theta_i = 1 / base**(2i/d), the pair
      rotation and its sign convention, and the inverse rotation.
* The HyperCache post again, Core Design, recompute paragraph, and the
  "15% CacheBlend" line of its Part A printout: the tokens with the largest
  layer-0 hidden-state drift are the ones recomputed.

Where the pages leave a step open, the plainest reading is taken; each such
reading is marked "Reading:" below.

Parity status of each function is stated in its docstring: "pinned by" names
the independent facts the CPU tests check it against.
"""

from __future__ import annotations

import numpy as np

HEAD_DIM = 128
E4M3_MAX = 448.0
INT4_QMAX = 7
FP16_MAX = 65504.0

FMT_FP8 = "fp8"
FMT_INT4 = "int4"
PAIRS_INTERLEAVED = "interleaved"
PAIRS_HALF_SPLIT = "half_split"


# ---------------------------------------------------------------------------
# Rounding to narrow binary formats
# ---------------------------------------------------------------------------

def round_to_format(x, p, emin):
    """Round float64 values to the binary format with a p-bit significand
    (hidden bit included) and smallest normal exponent `emin`, ties to even.

    Subnormals use the quantum 2**(emin - p + 1) of the smallest binade.
    Overflow is not handled here (the caller decides saturation vs inf).
    The sign, including that of zero, is kept.

    Exact: the scaling by a power of two and np.rint (round half to even)
    introduce no rounding of their own for p <= 53.

    Pinned by: equality with numpy's float32 cast (p=24), with Python's
    IEEE half packing (p=11) and torch's CPU bfloat16 cast (p=8).
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, e = np.frexp(ax)                 # ax = f * 2**e, f in [0.5, 1)
    lead = np.maximum(e - 1, emin)      # exponent of the leading bit, clamped
    qexp = lead - (p - 1)               # exponent of one unit in the last place
    n = np.rint(np.ldexp(ax, -qexp))    # exact scaling, then ties-to-even
    r = np.ldexp(n, qexp)
    return np.copysign(r, x)


def to_f32(x):
    """float64 -> fp32, round to nearest even (numpy's IEEE cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def f32_to_f16_value(x):
    """fp32 value -> fp16 value (float64 carrier), RNE, IEEE overflow to inf."""
    r = round_to_format(np.asarray(x, dtype=np.float32).astype(np.float64), 11, -14)
    return np.where(np.abs(r) > FP16_MAX, np.copysign(np.inf, r), r)


BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def f32_to_bf16_value(x):
    """fp32 value -> bfloat16 value (float64 carrier), RNE, IEEE overflow to inf."""
    r = round_to_format(np.asarray(x, dtype=np.float32).astype(np.float64), 8, -126)
    return np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, r), r)


def f16_bits(v):
    """Bits of fp16 values that are already exactly representable."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def bf16_bits(v):
    """Bits of bfloat16 values that are already exactly representable:
    the top half of their exact fp32 representation."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint32) << 16).astype(np.uint32).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# FP8 E4M3 (OCP "FN" flavour: no infinities, max 448, NaN = S.1111.111)
# ---------------------------------------------------------------------------
# Reading: the HyperCache post names only "E4M3".  The flavour with a finite
# maximum of 448 is taken because saturation at +-448 is the stated clamp.

def e4m3_value(code):
    """Decode E4M3FN codes to float64 from the format's definition:
    sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
    holds subnormals m/8 * 2**-6; S.1111.111 is NaN.

    Pinned by: torch's CPU float8_e4m3fn -> float32 conversion of all 256
    codes, and the format's landmarks (max 448, min normal 2**-6, min
    subnormal 2**-9)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6,
                   (1.0 + m / 8.0) * np.ldexp(1.0, (e - 7).astype(np.int64)))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(q):
    """Encode fp32 values to E4M3FN codes: round to nearest, ties to even
    mantissa, saturating every finite magnitude above 448 to 448 (code 0x7E),
    sign kept (so -0 and negatives that round to zero give 0x80).

    The value is first rounded to the E4M3 grid (4-bit significand, smallest
    normal exponent -6, subnormal quantum 2**-9); the rounded value is then
    written as sign / exponent / mantissa fields.

    Non-finite input is outside the contract; +-inf saturates like any large
    value and NaN maps to 0x7F / 0xFF.

    Pinned by: torch's CPU float8_e4m3fn cast on random and boundary fp32
    patterns, every rounding midpoint between adjacent codes, and the exact
    round trip of every representable value."""
    q = np.asarray(q, dtype=np.float32).astype(np.float64)
    neg = np.signbit(q)
    r = np.abs(round_to_format(q, 4, -6))
    r = np.where(r > E4M3_MAX, E4M3_MAX, r)          # saturation (also inf)
    is_nan = np.isnan(q)
    r = np.where(is_nan, 0.0, r)
    sub = r < 2.0 ** -6
    m_sub = np.rint(r / 2.0 ** -9).astype(np.int64)  # exact: r is on the grid
    safe = np.where(sub, 1.0, r)
    _, e = np.frexp(safe)
    lead = e - 1                                      # in [-6, 8]
    m_norm = np.rint(np.ldexp(safe, -(lead - 3)) - 8.0).astype(np.int64)
    code = np.where(sub, m_sub, ((lead + 7) << 3) | m_norm)
    code = np.where(is_nan, 0x7F, code)
    code = code | (neg.astype(np.int64) << 7)
    return code.astype(np.uint8)


# ---------------------------------------------------------------------------
# Per-vector scale and the two codecs
# ---------------------------------------------------------------------------
# Reading (group): one scale per 128-element head vector, i.e. per (layer,
# K|V, token, head).  Reading (scale): s = fp16_RNE(fp32(amax) / qmax) with an
# IEEE fp32 division, and the codes are computed with the stored fp16 s, which
# is the only scale a reader of the record sees.

def vector_amax(x):
    """max |x| over the last axis, in fp32 (exact)."""
    return np.max(np.abs(np.asarray(x, dtype=np.float32)), axis=-1)


def fp16_scale(amax, qmax):
    """fp16 scale value (float64 carrier) for each vector.

    s32 = fp32(amax) / qmax as an IEEE fp32 division, then fp16 RNE.
    Readings for the cases the pages leave open: amax == 0 gives s = 0;
    a positive amax whose scale underflows fp16 to zero gives the smallest
    fp16 subnormal 2**-24; a scale above the fp16 range gives 65504.

    Pinned by: the exact round trip of vectors whose scale is a power of two,
    and the worked byte/ratio figures of the HyperCache post."""
    amax = np.asarray(amax, dtype=np.float32)
    s32 = amax / np.float32(qmax)                     # IEEE fp32 division
    s = round_to_format(s32.astype(np.float64), 11, -14)
    s = np.where(s > FP16_MAX, FP16_MAX, s)
    s = np.where((s == 0) & (amax > 0), 2.0 ** -24, s)
    s = np.where(amax == 0, 0.0, s)
    return s


def _quotient_f32(x, s):
    """fp32(x) / fp32(s) as an IEEE fp32 division; where s == 0 (all-zero
    vector) the element itself (a signed zero) stands in for the quotient."""
    x = np.asarray(x, dtype=np.float32)
    s32 = np.asarray(s, dtype=np.float64).astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = x / np.where(s32 == 0, np.float32(1.0), s32)
    return np.where(s32 == 0, x, q)


def quant_fp8_vectors(x):
    """FP8 put of head vectors x[..., 128] (fp32-exact values).

    Returns (codes uint8 [..., 128], scale value float64 [...]).
    Pinned by: exact round trip of representable vectors; encoder pins."""
    amax = vector_amax(x)
    s = fp16_scale(amax, E4M3_MAX)
    q = _quotient_f32(x, s)
    return e4m3_encode(q), s


def quant_int4_vectors(x):
    """INT4 grouped symmetric put of head vectors x[..., 128].

    q_j = clamp(rint(fp32(x_j) / fp32(s)), -7, 7) with s = fp16(amax / 7);
    element 2k goes to the low nibble of byte k, element 2k+1 to the high
    nibble, two's complement.
    Reading: symmetric means codes in [-7, 7] (-8 is never produced).

    Returns (packed uint8 [..., 64], scale value float64 [...]).
    Pinned by: brute force over small integer grids, exact round trip of
    q * 2**k vectors, and every rounding midpoint."""
    amax = vector_amax(x)
    s = fp16_scale(amax, INT4_QMAX)
    q = _quotient_f32(x, s).astype(np.float64)
    qi = np.clip(np.rint(q), -INT4_QMAX, INT4_QMAX).astype(np.int64)
    lo = qi[..., 0::2] & 0xF
    hi = qi[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8), s


def int4_unpack(packed):
    """Packed bytes [..., 64] -> signed integers [..., 128]."""
    p = np.asarray(packed, dtype=np.int64)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# ---------------------------------------------------------------------------
# Records: one per (layer, logical block)
# ---------------------------------------------------------------------------
# Layout (ours; the pages do not print one):
#   [K codes][V codes][K scales][V scales]
# codes ordered token-major, then head, then element; scales are fp16,
# little endian, ordered token-major then head.

def code_bytes_per_vector(fmt, head_dim=HEAD_DIM):
    return head_dim if fmt == FMT_FP8 else head_dim // 2


def record_bytes(fmt, block_tokens, n_kv_heads, head_dim=HEAD_DIM):
    """Bytes of one (layer, block) record: codes plus one 2-byte scale per
    vector, for K and V.  KV-handoff module, section 1: KV bytes are
    2 * layers * kv_heads * head_dim * tokens * bytes_per_element; here the
    element width is that of the code, plus the scales.

    Pinned by: the HyperCache post's Part B figures (1.97x, 3.88x and the
    byte counts of its FP8 frame and INT4 file less their headers)."""
    n = block_tokens * n_kv_heads
    return 2 * n * code_bytes_per_vector(fmt, head_dim) + 2 * n * 2


def assemble_records(k_codes, v_codes, k_scales, v_scales):
    """Codes [..., T_b, H, cb] and scale values [..., T_b, H] -> uint8 records
    [..., record_bytes]."""
    lead = k_codes.shape[:-3]
    flat = lambda a: a.reshape(lead + (-1,))
    ks = f16_bits(k_scales).astype("<u2").view(np.uint8)
    vs = f16_bits(v_scales).astype("<u2").view(np.uint8)
    ks = ks.reshape(lead + (-1,))
    vs = vs.reshape(lead + (-1,))
    return np.concatenate([flat(k_codes), flat(v_codes), ks, vs], axis=-1).astype(np.uint8)


def split_records(rec, fmt, block_tokens, n_kv_heads, head_dim=HEAD_DIM):
    """Inverse of assemble_records: returns (k_codes, v_codes, k_scale, v_scale)
    with scale values as float64."""
    cb = code_bytes_per_vector(fmt, head_dim)
    n = block_tokens * n_kv_heads
    lead = rec.shape[:-1]
    shp = lead + (block_tokens, n_kv_heads, cb)
    kc = rec[..., 0:n * cb].reshape(shp)
    vc = rec[..., n * cb:2 * n * cb].reshape(shp)
    base = 2 * n * cb
    ks = np.ascontiguousarray(rec[..., base:base + 2 * n]).view("<u2").reshape(lead + (block_tokens, n_kv_heads))
    vs = np.ascontiguousarray(rec[..., base + 2 * n:base + 4 * n]).view("<u2").reshape(lead + (block_tokens, n_kv_heads))
    ksv = ks.astype(np.uint16).view(np.float16).astype(np.float64)
    vsv = vs.astype(np.uint16).view(np.float16).astype(np.float64)
    return kc, vc, ksv, vsv


def put(k_pages, v_pages, block_table, fmt):
    """Quantize blocks gathered from a paged buffer into records.

    k_pages, v_pages: [L, P, T_b, H, 128] source values (any float dtype; they
    are taken at their exact fp32 value).  block_table: [n_blocks] int, logical
    block -> page; entries that are negative or not below the page count are
    skipped (reading: a negative entry marks a block to skip, and an entry
    past the buffer is never dereferenced).
    Returns (records uint8 [L, n_blocks, rec_bytes], written bool [n_blocks]);
    records of skipped blocks are all zero.
    """
    L, P, T_b, H, d = k_pages.shape
    assert d == HEAD_DIM
    table = np.asarray(block_table, dtype=np.int64)
    nb = table.shape[0]
    rb = record_bytes(fmt, T_b, H, d)
    out = np.zeros((L, nb, rb), dtype=np.uint8)
    live = (table >= 0) & (table < P)
    if not live.any():
        return out, live                     # every block skipped: nothing written
    pages = table[live]
    quant = quant_fp8_vectors if fmt == FMT_FP8 else quant_int4_vectors
    kx = np.ascontiguousarray(np.asarray(k_pages)[:, pages], dtype=np.float32)
    vx = np.ascontiguousarray(np.asarray(v_pages)[:, pages], dtype=np.float32)
    kc, ks = quant(kx)
    vc, vs = quant(vx)
    out[:, live] = assemble_records(kc, vc, ks, vs)
    return out, live


def dequant_records(records, fmt, block_tokens, n_kv_heads):
    """Records [..., rec_bytes] -> (K, V) float64 [..., T_b, H, 128].
    Dequantization code * scale is exact in float64 (and in fp32)."""
    kc, vc, ks, vs = split_records(records, fmt, block_tokens, n_kv_heads)
    if fmt == FMT_FP8:
        kv = e4m3_value(kc)
        vv = e4m3_value(vc)
    else:
        kv = int4_unpack(kc).astype(np.float64)
        vv = int4_unpack(vc).astype(np.float64)
    return kv * ks[..., None], vv * vs[..., None]


# ---------------------------------------------------------------------------
# RoPE (KV-handoff module listing; HyperCache post, relative-RoPE paragraph)
# ---------------------------------------------------------------------------

def rope_theta(base, head_dim=HEAD_DIM):
    """theta_i = 1 / base**(2i/d), i = 0 .. d/2 - 1, in float64, written as the
    KV-handoff module's rope_cache writes it.

    Pinned by: theta_0 = 1, a constant ratio base**(-2/d) between neighbours,
    and the relative-position property of RoPE scores."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return 1.0 / (float(base) ** (2.0 * i / head_dim))


def pair_indices(pairs, head_dim=HEAD_DIM):
    """Element indices (a_i, b_i) of rotation pair i.

    interleaved: (2i, 2i+1), the KV-handoff module's apply_rope convention.
    half_split:  (i, i + d/2), the split-halves convention.
    Reading: the pages print only the interleaved form; the half-split form is
    the same rotation applied to a permuted vector."""
    i = np.arange(head_dim // 2)
    if pairs == PAIRS_INTERLEAVED:
        return 2 * i, 2 * i + 1
    if pairs == PAIRS_HALF_SPLIT:
        return i, i + head_dim // 2
    raise ValueError(pairs)


def rotate_pairs(x, angle, pairs):
    """Rotate every pair of x[..., d] by angle[..., d/2]:
    (a, b) -> (a cos - b sin, a sin + b cos), the sign convention of the
    KV-handoff module's apply_rope.

    cos and sin are computed in float64 and the arithmetic is done in x's
    dtype: float64 for the oracle proper; float32 only to replay the
    HyperCache post's float32 experiment."""
    x = np.asarray(x)
    ia, ib = pair_indices(pairs, x.shape[-1])
    c = np.cos(np.asarray(angle, dtype=np.float64)).astype(x.dtype)
    s = np.sin(np.asarray(angle, dtype=np.float64)).astype(x.dtype)
    a = x[..., ia]
    b = x[..., ib]
    out = np.empty_like(x)
    out[..., ia] = a * c - b * s
    out[..., ib] = a * s + b * c
    return out


def rope_apply(x, pos, base, pairs):
    """RoPE at integer positions pos[T] of x[T, H, d] (pos -> angle pos*theta_i)."""
    th = rope_theta(base, x.shape[-1])
    ang = np.asarray(pos, dtype=np.float64)[:, None] * th[None, :]
    return rotate_pairs(x, ang[:, None, :], pairs)


def rope_strip(x, pos, base, pairs):
    """Inverse of rope_apply: rotate by -pos (KV-handoff module, strip_rope)."""
    th = rope_theta(base, x.shape[-1])
    ang = -np.asarray(pos, dtype=np.float64)[:, None] * th[None, :]
    return rotate_pairs(x, ang[:, None, :], pairs)


def rope_shift(x, delta_m, base, pairs):
    """Relative shift of post-RoPE keys by delta_m = m_new - m_old (HyperCache
    post, SO(2) identity R(m_new th) = R(dm th) R(m_old th)).  delta_m is a
    scalar or broadcasts against x's leading axes (one value per block).

    Pinned by: the HyperCache post's float32 shift error 4.77e-07 for
    1024 -> 8192, dm = 0 identity, composition, norm preservation, and
    equality with strip-then-apply."""
    th = rope_theta(base, x.shape[-1])
    dm = np.asarray(delta_m, dtype=np.float64)
    ang = dm[..., None] * th
    return rotate_pairs(x, ang, pairs)


# ---------------------------------------------------------------------------
# Fetch: dequantize, shift K, convert, scatter into pages
# ---------------------------------------------------------------------------

DTYPES = ("f32", "f16", "bf16")


def round_output(y, dtype):
    """float64 -> stored output value (float64 carrier): RNE to fp32, then RNE
    to fp16 / bf16 when that is the page dtype."""
    f = to_f32(y)
    if dtype == "f32":
        return f.astype(np.float64)
    if dtype == "f16":
        return f32_to_f16_value(f)
    if dtype == "bf16":
        return f32_to_bf16_value(f)
    raise ValueError(dtype)


def fetch_exact(records, fmt, block_tokens, n_kv_heads, delta_m, base, pairs):
    """Unrounded fetch result per logical block: (K, V) float64
    [L, n_blocks, T_b, H, 128].  V is dequantized only; K is dequantized and
    shifted by its delta: delta_m is [n_blocks] (one delta per block) or
    [n_blocks, T_b] (one per token, e.g. -m to strip the cached phase as the
    KV-handoff module's strip_rope does)."""
    kd, vd = dequant_records(records, fmt, block_tokens, n_kv_heads)
    dm = np.asarray(delta_m, dtype=np.float64)
    dm = dm[None, :, None, None] if dm.ndim == 1 else dm[None, :, :, None]
    kr = rope_shift(kd, dm, base, pairs)
    return kr, vd


def fetch(records, fmt, block_tokens, n_kv_heads, block_table, delta_m, base,
          pairs, k_pages, v_pages, out_dtype):
    """Fetch into page arrays k_pages, v_pages [L, P, T_b, H, 128] (float64
    carriers of the page dtype, modified in place).  Blocks whose table entry
    is negative or not below the page count are skipped; pages that no block
    names keep their contents."""
    table = np.asarray(block_table, dtype=np.int64)
    live = (table >= 0) & (table < k_pages.shape[1])
    kr, vd = fetch_exact(records[:, live], fmt, block_tokens, n_kv_heads,
                         np.asarray(delta_m)[live], base, pairs)
    k_pages[:, table[live]] = round_output(kr, out_dtype)
    v_pages[:, table[live]] = round_output(vd, out_dtype)
    return k_pages, v_pages


# ---------------------------------------------------------------------------
# CRC-32 (the common zlib / ISO-HDLC variant)
# ---------------------------------------------------------------------------
# Reading: the HyperCache post says only "CRC32"; the ubiquitous variant is
# taken (reflected polynomial 0xEDB88320, initial value and final xor
# 0xFFFFFFFF), computed over the whole record.

def crc32_table():
    """Byte table built bit by bit from the reflected polynomial."""
    t = np.zeros(256, dtype=np.uint32)
    for n in range(256):
        c = n
        for _ in range(8):
            c = (c >> 1) ^ 0xEDB88320 if (c & 1) else (c >> 1)
        t[n] = c
    return t


def crc32_bitwise(data: bytes) -> int:
    """Bit-at-a-time CRC-32, for small inputs."""
    c = 0xFFFFFFFF
    for byte in data:
        c ^= byte
        for _ in range(8):
            c = (c >> 1) ^ 0xEDB88320 if (c & 1) else (c >> 1)
    return c ^ 0xFFFFFFFF


def crc32_records(records):
    """CRC-32 of each record: records uint8 [..., nbytes] -> uint32 [...].
    Byte-table form, vectorised across records.

    Pinned by: the check value 0xCBF43926 of b"123456789", zlib.crc32 on
    random data, and equality with the bit-at-a-time form."""
    rec = np.asarray(records, dtype=np.uint8)
    lead = rec.shape[:-1]
    cols = np.ascontiguousarray(rec.reshape(-1, rec.shape[-1]).T)
    table = crc32_table()
    c = np.full(cols.shape[1], 0xFFFFFFFF, dtype=np.uint32)
    for j in range(cols.shape[0]):
        c = table[(c ^ cols[j]) & 0xFF] ^ (c >> np.uint32(8))
    return (c ^ np.uint32(0xFFFFFFFF)).reshape(lead)


def kv_bytes(layers, kv_heads, head_dim, tokens, bytes_per_elem):
    """KV bytes = 2 * layers * kv_heads * head_dim * tokens * bytes_per_element
    (KV-handoff module, section 1)."""
    return 2 * layers * kv_heads * head_dim * tokens * bytes_per_elem


# ---------------------------------------------------------------------------
# Recompute selection after a chunk reorder (the CacheBlend step)
# ---------------------------------------------------------------------------
# The HyperCache post, Core Design, recompute paragraph: layer 0's KV is exact
# after the rotation, and the tokens whose layer-0 hidden state drifts the
# most, about 15% of them, are recomputed through the deeper layers.  Part A
# of its printout reports the "15% CacheBlend" configuration.
# Reading: the drift of token t is the Euclidean norm of the difference of
# its two layer-0 hidden states (fresh context minus cached context); the
# selection is the k largest drifts, ties going to the lower token index and
# NaN ranking above every number; +0 and -0 are equal.  The list is returned
# in increasing token order (the order a recompute pass gathers them in).

def token_drift(h_cached, h_fresh):
    """Per-token drift ||h_fresh[t] - h_cached[t]||_2 over the last axis, in
    float64 (inputs of any binary format convert exactly).

    Pinned by: Pythagorean rows with integer norms, math.hypot row by row on
    random data, symmetry, zero for equal rows, exact scaling by powers of
    two, and the triangle inequality."""
    a = np.asarray(h_cached, dtype=np.float64)
    b = np.asarray(h_fresh, dtype=np.float64)
    d = b - a
    return np.sqrt(np.sum(d * d, axis=-1))


def recompute_count(n_tokens, percent=15):
    """Reading: k = floor(percent * n / 100) tokens are recomputed (the post
    says "about 15%").

    Pinned by: small cases written out, and k / n within 1 / n of 15%."""
    return (int(n_tokens) * int(percent)) // 100


def select_top_tokens(drift, k):
    """Indices (int32, increasing) of the k tokens with the largest drift.

    Order: larger value first; NaN above everything; equal values (+0 and
    -0 included) by lower index.  k must lie in [0, n].

    Pinned by: a brute-force search over all k-subsets of tiny inputs for
    the set that outranks its complement, and worked cases (all equal,
    k = 0, k = n, NaN, signed zeros, negative values)."""
    v = np.asarray(drift, dtype=np.float64).reshape(-1)
    n = v.size
    if not 0 <= k <= n:
        raise ValueError(f"k={k} outside [0, {n}]")
    nan = np.isnan(v)
    value = np.where(nan, 0.0, v)
    # np.lexsort: the last key is the primary one, each ascending
    ranked = np.lexsort((np.arange(n), -value, ~nan))
    return np.sort(ranked[:k]).astype(np.int32)


# ---------------------------------------------------------------------------
# Self-describing frames (record container)
# ---------------------------------------------------------------------------
# The HyperCache post's FP8 wire frame and INT4 disk file carry headers of 68
# and 69 bytes around the payload (Part B byte counts) whose layout it does not
# give.  Reading: a 64-byte little-endian header of our own precedes each
# record, so a frame names its shape, its place in the cache and the cached
# position of its first token (what a reader needs for the relative shift
# dm = m_new - m_old), and carries the record's CRC-32 and a CRC-32 of the
# header itself:
#    0 u32 magic 0x46564B48 ("HKVF")   4 u16 version 1   6 u16 header bytes 64
#    8 u8 format (0 FP8, 1 INT4)       9 u8 zero         10 u16 head_dim
#   12 u16 block_tokens               14 u16 n_kv_heads
#   16 u32 layer   20 u32 block   24 i32 m_old   28 u32 payload bytes
#   32 u32 payload CRC-32   36..59 zero   60 u32 CRC-32 of bytes 0..59

FRAME_HEADER_BYTES = 64
FRAME_MAGIC = 0x46564B48
FRAME_VERSION = 1
# verification flags
FRAME_BAD_MAGIC = 1
FRAME_BAD_HEADER_CRC = 2
FRAME_BAD_GEOMETRY = 4
FRAME_BAD_INDEX = 8
FRAME_BAD_PAYLOAD_CRC = 16


def _u32(b, off):
    return int(b[off]) | int(b[off + 1]) << 8 | int(b[off + 2]) << 16 | int(b[off + 3]) << 24


def _put_u(b, off, value, n):
    for j in range(n):
        b[off + j] = (int(value) >> (8 * j)) & 0xFF


def frame_header(fmt, block_tokens, n_kv_heads, layer, block, m_old, payload_bytes,
                 payload_crc, head_dim=HEAD_DIM):
    """The 64 header bytes of one frame (uint8 [64]).

    Pinned by: a header spelled out byte by byte from the layout above, the
    header CRC against zlib, and parse_frame_header round trips."""
    b = np.zeros(FRAME_HEADER_BYTES, dtype=np.uint8)
    _put_u(b, 0, FRAME_MAGIC, 4)
    _put_u(b, 4, FRAME_VERSION, 2)
    _put_u(b, 6, FRAME_HEADER_BYTES, 2)
    b[8] = 0 if fmt == FMT_FP8 else 1
    _put_u(b, 10, head_dim, 2)
    _put_u(b, 12, block_tokens, 2)
    _put_u(b, 14, n_kv_heads, 2)
    _put_u(b, 16, layer, 4)
    _put_u(b, 20, block, 4)
    _put_u(b, 24, int(m_old) & 0xFFFFFFFF, 4)
    _put_u(b, 28, payload_bytes, 4)
    _put_u(b, 32, payload_crc, 4)
    _put_u(b, 60, int(crc32_records(b[None, :60])[0]), 4)
    return b


def parse_frame_header(b):
    """Field dictionary of a 64-byte header (no checks)."""
    b = np.asarray(b, dtype=np.uint8)
    m_old = _u32(b, 24)
    return {
        "magic": _u32(b, 0), "version": int(b[4]) | int(b[5]) << 8,
        "header_bytes": int(b[6]) | int(b[7]) << 8, "format": int(b[8]),
        "head_dim": int(b[10]) | int(b[11]) << 8,
        "block_tokens": int(b[12]) | int(b[13]) << 8,
        "n_kv_heads": int(b[14]) | int(b[15]) << 8,
        "layer": _u32(b, 16), "block": _u32(b, 20),
        "m_old": m_old - (1 << 32) if m_old >= 1 << 31 else m_old,
        "payload_bytes": _u32(b, 28), "payload_crc": _u32(b, 32),
        "header_crc": _u32(b, 60),
    }


def make_frames(records, fmt, block_tokens, n_kv_heads, m_old, layer_base=0):
    """Frames [L, n_blocks, 64 + record bytes] for records [L, n_blocks, bytes]
    and the cached positions m_old [n_blocks] (shared by the layers)."""
    rec = np.asarray(records, dtype=np.uint8)
    L, nb, rb = rec.shape
    crc = crc32_records(rec)
    out = np.zeros((L, nb, FRAME_HEADER_BYTES + rb), dtype=np.uint8)
    for l in range(L):
        for b in range(nb):
            out[l, b, :FRAME_HEADER_BYTES] = frame_header(
                fmt, block_tokens, n_kv_heads, layer_base + l, b, int(m_old[b]), rb,
                int(crc[l, b]))
    out[:, :, FRAME_HEADER_BYTES:] = rec
    return out


def verify_frames(frames, fmt, block_tokens, n_kv_heads, layer_base=0):
    """Flags per frame (uint32 [L, n_blocks]); 0 means the frame is intact and
    belongs at (layer_base + l, b) of a cache of this shape and format.

    Pinned by: intact frames give 0; each kind of damage (magic, a header
    field, the header CRC word, a payload byte, a frame moved to another
    slot) raises its own flag."""
    fr = np.asarray(frames, dtype=np.uint8)
    L, nb, _ = fr.shape
    rb = record_bytes(fmt, block_tokens, n_kv_heads)
    payload_crc = crc32_records(fr[:, :, FRAME_HEADER_BYTES:FRAME_HEADER_BYTES + rb])
    head_crc = crc32_records(fr[:, :, :60])
    out = np.zeros((L, nb), dtype=np.uint32)
    for l in range(L):
        for b in range(nb):
            h = parse_frame_header(fr[l, b, :FRAME_HEADER_BYTES])
            f = 0
            if (h["magic"], h["version"], h["header_bytes"]) != \
                    (FRAME_MAGIC, FRAME_VERSION, FRAME_HEADER_BYTES):
                f |= FRAME_BAD_MAGIC
            if h["header_crc"] != int(head_crc[l, b]):
                f |= FRAME_BAD_HEADER_CRC
            if (h["format"], h["head_dim"], h["block_tokens"], h["n_kv_heads"],
                    h["payload_bytes"]) != (0 if fmt == FMT_FP8 else 1, HEAD_DIM, block_tokens,
                                            n_kv_heads, rb):
                f |= FRAME_BAD_GEOMETRY
            if (h["layer"], h["block"]) != (layer_base + l, b):
                f |= FRAME_BAD_INDEX
            if h["payload_crc"] != int(payload_crc[l, b]):
                f |= FRAME_BAD_PAYLOAD_CRC
            out[l, b] = f
    return out


def frame_delta_m(frames, m_new):
    """dm[b] = m_new[b] - m_old of the first layer's frame b (the relative
    shift of the HyperCache post's relative-RoPE paragraph), clamped to int32."""
    fr = np.asarray(frames, dtype=np.uint8)
    m_old = np.array([parse_frame_header(fr[0, b, :FRAME_HEADER_BYTES])["m_old"]
                      for b in range(fr.shape[1])], dtype=np.int64)
    d = np.asarray(m_new, dtype=np.int64) - m_old
    return np.clip(d, -(1 << 31), (1 << 31) - 1).astype(np.int32)
