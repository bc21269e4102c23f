"""Pins of the oracle's per-vector scale, FP8 and INT4 puts, records and byte
accounting: exact round trips, brute force on small integer grids, torch
cross-checks, and the byte counts and ratios printed on the pages."""
import numpy as np
import torch

import oracle as O
from conftest import load_golden


def _vec(rng, n=1):
    return rng.standard_normal((n, 128)).astype(np.float32)


def test_fp8_round_trip_of_representable_vectors():
    """x = c * 2**k with c on the E4M3 grid and one |c| = 448: the scale is
    exactly 2**k, the codes are c and dequantization restores x."""
    rng = np.random.default_rng(21)
    grid = O.e4m3_value(np.array([c for c in range(256) if c not in (0x7F, 0xFF)]))
    for k in range(-15, 8):
        c = rng.choice(grid, size=(4, 128))
        c[:, rng.integers(0, 128)] = 448.0 * rng.choice([-1, 1])
        x = (c * 2.0 ** k).astype(np.float32)
        assert np.array_equal(x.astype(np.float64), c * 2.0 ** k)
        codes, s = O.quant_fp8_vectors(x)
        assert np.all(s == 2.0 ** k)
        assert np.array_equal(O.e4m3_value(codes), c)


def test_fp8_put_matches_torch_pipeline():
    """Same steps through torch's own fp32 division, fp16 cast and fp8 cast."""
    rng = np.random.default_rng(22)
    x = (_vec(rng, 4096) * np.exp(rng.uniform(-6, 6, (4096, 1)))).astype(np.float32)
    codes, s = O.quant_fp8_vectors(x)
    t = torch.from_numpy(x)
    amax = t.abs().amax(dim=1, keepdim=True)
    st = (amax / 448.0).to(torch.float16).float()
    q = (t / st).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(s, st.numpy()[:, 0].astype(np.float64))
    assert np.array_equal(codes, q)


def test_scale_edge_cases():
    z = np.zeros((1, 128), np.float32)
    z[0, 5] = -0.0
    codes, s = O.quant_fp8_vectors(z)
    assert s[0] == 0.0 and codes[0, 0] == 0x00 and codes[0, 5] == 0x80
    ic, isc = O.quant_int4_vectors(z)
    assert isc[0] == 0.0 and np.all(ic == 0)
    tiny = np.full((1, 128), 1e-30, np.float32)
    _, s = O.quant_fp8_vectors(tiny)
    assert s[0] == 2.0 ** -24
    huge = np.full((1, 128), 1e30, np.float32)
    codes, s = O.quant_fp8_vectors(huge)
    assert s[0] == 65504.0 and np.all(codes == 0x7E)
    codes, s = O.quant_fp8_vectors(-huge)
    assert np.all(codes == 0xFE)


def test_int4_round_trip_and_packing():
    rng = np.random.default_rng(23)
    for k in range(-20, 12):
        q = rng.integers(-7, 8, size=(8, 128))
        q[:, 3] = 7 * rng.choice([-1, 1], size=8)
        x = (q * 2.0 ** k).astype(np.float32)
        packed, s = O.quant_int4_vectors(x)
        assert np.all(s == 2.0 ** k)
        assert np.array_equal(O.int4_unpack(packed), q)
    x = np.zeros((1, 128), np.float32)
    x[0, 0], x[0, 1], x[0, 2], x[0, 3] = 7.0, -1.0, -7.0, 3.0
    packed, _ = O.quant_int4_vectors(x)
    assert packed[0, 0] == 0xF7 and packed[0, 1] == 0x39


def test_int4_midpoints_round_half_to_even():
    """(n + 1/2) * s for n = -7..6 lands on the even neighbour."""
    n = np.arange(-7, 7)
    x = np.zeros((n.size, 128), np.float32)
    x[:, 0] = 7.0                       # s = 1 exactly
    x[:, 1] = n + 0.5
    packed, s = O.quant_int4_vectors(x)
    assert np.all(s == 1.0)
    got = O.int4_unpack(packed)[:, 1]
    want = np.where(n % 2 == 0, n, n + 1)
    assert np.array_equal(got, want)


def test_int4_matches_torch_pipeline_brute_force():
    rng = np.random.default_rng(24)
    x = (_vec(rng, 8192) * np.exp(rng.uniform(-8, 8, (8192, 1)))).astype(np.float32)
    packed, s = O.quant_int4_vectors(x)
    t = torch.from_numpy(x)
    st = (t.abs().amax(dim=1, keepdim=True) / 7.0).to(torch.float16).float()
    q = torch.round(t / st).clamp(-7, 7).to(torch.int64).numpy()   # half to even
    assert np.array_equal(s, st.numpy()[:, 0].astype(np.float64))
    assert np.array_equal(O.int4_unpack(packed), q)


def test_int4_cosine_supports_symmetric_seven_levels():
    """Statistical support (not a pin) for codes in [-7, 7]: on standard
    normal data the cosine is nearer the HyperCache post's INT4 figure with
    qmax 7 than with qmax 8."""
    g = load_golden("hypercache_part_b.json")["int4_cosine"]
    x = np.random.default_rng(0).standard_normal((4096, 128)).astype(np.float32)
    packed, s = O.quant_int4_vectors(x)
    y = O.int4_unpack(packed) * s[:, None]
    cos7 = np.sum(x * y) / np.sqrt(np.sum(x * x) * np.sum(y * y))
    s8 = (np.abs(x).max(1) / 8).astype(np.float16).astype(np.float64)
    y8 = np.clip(np.rint(x / s8[:, None]), -8, 7) * s8[:, None]
    cos8 = np.sum(x * y8) / np.sqrt(np.sum(x * x) * np.sum(y8 * y8))
    assert abs(cos7 - g) < abs(cos8 - g)
    assert abs(cos7 - g) < 1e-3


def test_record_bytes_reproduce_printed_ratios_and_sizes():
    g = load_golden("hypercache_part_b.json")
    fp16_vec = 128 * 2
    fp8_vec = O.record_bytes(O.FMT_FP8, 1, 1) // 2
    int4_vec = O.record_bytes(O.FMT_INT4, 1, 1) // 2
    assert (fp8_vec, int4_vec) == (130, 66)
    assert round(fp16_vec / fp8_vec, 2) == g["fp8_e4m3_compression"]
    assert round(fp16_vec / int4_vec, 2) == g["int4_grouped_compression"]
    # 1,024 head vectors (64 tokens x 8 heads x K,V): payload plus a small
    # header gives the printed frame / file sizes.
    fp8_payload = O.record_bytes(O.FMT_FP8, 64, 8)
    int4_payload = O.record_bytes(O.FMT_INT4, 64, 8)
    assert (fp8_payload, int4_payload) == (133120, 67584)
    assert 0 < g["tcp_fetch_frame_bytes"] - fp8_payload < 128
    assert 0 < g["int4_hckv_bytes_on_disk"] - int4_payload < 128


def test_kv_bytes_formula_matches_handoff_module():
    g = load_golden("kv_handoff_bytes.json")
    m = g["qwen3_8b"]
    per_tok = O.kv_bytes(m["layers"], m["kv_heads"], m["head_dim"], 1, 2)
    assert per_tok == g["fp16_bytes_per_token_kib"] * 1024
    assert round(O.kv_bytes(m["layers"], m["kv_heads"], m["head_dim"], 32768, 2) / 2 ** 30, 1) \
        == g["fp16_32k_context_gib"]
    assert O.kv_bytes(m["layers"], m["kv_heads"], m["head_dim"], 25000, 2) == g["fp16_25k_context_bytes"]
    assert round(O.kv_bytes(m["layers"], m["kv_heads"], m["head_dim"], 25000, 1) / 2 ** 30, 2) \
        == g["int8_25k_context_gib"]
    for name, b in (("int8", 1), ("int4", 0.5)):
        assert O.kv_bytes(m["layers"], m["kv_heads"], m["head_dim"], 1, b) \
            == g["checklist_kib_per_token"][name] * 1024
    # with one fp16 scale per 128-element vector the codec's record bytes per
    # token are the codes plus 2 B per vector
    per_tok_fp8 = m["layers"] * O.record_bytes(O.FMT_FP8, 1, m["kv_heads"])
    assert per_tok_fp8 == 72 * 1024 + 2 * 2 * m["layers"] * m["kv_heads"]


def test_records_split_inverts_assemble():
    rng = np.random.default_rng(25)
    for fmt in (O.FMT_FP8, O.FMT_INT4):
        cb = O.code_bytes_per_vector(fmt)
        kc = rng.integers(0, 256, (2, 3, 16, 8, cb)).astype(np.uint8)
        vc = rng.integers(0, 256, (2, 3, 16, 8, cb)).astype(np.uint8)
        ks = rng.standard_normal((2, 3, 16, 8)).astype(np.float16).astype(np.float64)
        vs = rng.standard_normal((2, 3, 16, 8)).astype(np.float16).astype(np.float64)
        rec = O.assemble_records(kc, vc, ks, vs)
        assert rec.shape == (2, 3, O.record_bytes(fmt, 16, 8))
        a, b, c, d = O.split_records(rec, fmt, 16, 8)
        assert np.array_equal(a, kc) and np.array_equal(b, vc)
        assert np.array_equal(c, ks) and np.array_equal(d, vs)
        # layout: K codes first, then V codes, then K scales, then V scales
        assert np.array_equal(rec[0, 0, :cb], kc[0, 0, 0, 0])
        assert rec[0, 0, 2 * 16 * 8 * cb:2 * 16 * 8 * cb + 2].view("<u2")[0] == \
            np.float16(ks[0, 0, 0, 0]).view(np.uint16)
