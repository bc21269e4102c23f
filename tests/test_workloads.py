"""Host logic of the seeded workloads: shapes, reproducibility, tables and
deltas (no arithmetic of the method lives there)."""
import numpy as np

from quantization_rope_reuse_amd import workloads as W


def test_shapes_and_byte_sizes():
    assert W.TINY.n_blocks == 4 and W.GQA_REORDER.n_blocks == 84
    assert W.QWEN3_8B.n_blocks == 512 and W.LLAMA3_70B.n_blocks == 1024
    assert W.INT4_L3.n_blocks == 256
    # fp16 Qwen3-8B-shaped cache is 4.5 GiB; bf16 Llama-3-70B-shaped ~21.5 GB
    assert W.QWEN3_8B.n_vectors * 2 * 128 * 2 == int(4.5 * 2 ** 30)
    assert W.LLAMA3_70B.n_vectors * 2 * 128 * 2 == 21474836480


def test_reorder_plan():
    old, dm = W.reorder_plan(W.GQA_REORDER)
    vals, counts = np.unique(dm, return_counts=True)
    assert dict(zip(vals.tolist(), counts.tolist())) == {-512: 32, 0: 20, 512: 32}
    assert sorted(old.tolist()) == list(range(84))
    assert dm[:16].tolist() == [0] * 16 and dm[-4:].tolist() == [0] * 4
    assert old[16] == (256 + 512) // 16 and old[48] == 256 // 16


def test_tables_are_permutations_and_deltas_in_range():
    for w in W.ALL:
        for t in (W.put_table(w), W.fetch_table(w)):
            assert sorted(t.tolist()) == list(range(w.n_blocks))
        d = W.delta_m(w)
        assert d.shape == (w.n_blocks,) and d.dtype == np.int32
        if w.delta_kind == "uniform":
            assert d.min() >= -w.delta_value and d.max() <= w.delta_value
            assert d.min() < 0 < d.max()
    assert np.all(W.delta_m(W.LLAMA3_70B) == 8192)
    assert np.all(W.delta_m(W.TINY) == 7168)


def test_host_values_reproducible_and_outliers():
    w = W.INT4_L3
    a = W.host_layer_values(w, 3, 0)
    b = W.host_layer_values(w, 3, 0)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, W.host_layer_values(w, 3, 1))
    ch = W.outlier_channels(w, 3)
    assert ch.size == 10
    flat = a.reshape(w.n_tokens, -1)
    big = np.abs(flat[:, ch]).mean()
    rest = np.abs(np.delete(flat, ch, axis=1)).mean()
    assert 15 < big / rest < 25


def test_tiny_values():
    k, v = W.tiny_pre_rope_kv()
    g = np.random.default_rng(0)
    assert np.array_equal(k, g.standard_normal((64, 8, 128)).astype(np.float32))
    assert W.tiny_positions()[0] == 1024 and W.tiny_positions()[-1] == 1087


def test_pages_from_tokens():
    w = W.TINY
    x = np.arange(64 * 8 * 128, dtype=np.float32).reshape(64, 8, 128)
    t = np.array([2, 0, 3, 1])
    p = W.pages_from_tokens(x, w, t)
    assert np.array_equal(p[2], x[0:16]) and np.array_equal(p[1], x[48:64])


def test_drift_workloads():
    assert [w.n_tokens for w in W.DRIFT_ALL] == [1280, 32768, 65536]
    w = W.DRIFT_GQA
    s = W.drift_sigma(w)
    assert not s[:w.lead_tokens].any() and (s[w.lead_tokens:] > 0).all()
    # largest right after a chunk boundary, on average
    j = (np.arange(w.n_tokens) - w.lead_tokens) % w.chunk_tokens
    body = s[w.lead_tokens:]
    jj = j[w.lead_tokens:]
    assert body[jj < 16].mean() > 3 * body[jj > 256].mean()
    c, f = W.host_hidden_states(w)
    c2, f2 = W.host_hidden_states(w)
    assert np.array_equal(c, c2) and np.array_equal(f, f2)
    assert c.shape == (1280, 4096) and c.dtype == np.float32
    assert np.array_equal(c[:w.lead_tokens], f[:w.lead_tokens])
    assert (np.abs(f - c)[w.lead_tokens:].max(axis=1) > 0).all()


def test_drift_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, 1.0 + 2.0**-9, -2.5e-3], np.float32)
    got = W._round_dtype(x, "bf16")
    assert got.tolist()[:4] == [1.0, 1.0, 1.0 + 2.0**-6, 1.0]
    assert (got.view(np.uint32) & 0xFFFF == 0).all()
    assert abs(got[4] - x[4]) <= 2.0**-9 * abs(x[4])


def test_block_positions():
    for w in W.ALL:
        m_old, m_new = W.block_positions(w)
        assert np.array_equal(m_new.astype(np.int64) - m_old, W.delta_m(w))
        assert m_new.min() >= 0 and m_old.min() >= 0
    m_old, m_new = W.block_positions(W.GQA_REORDER)
    # DocB's first block sat after Sys + DocA in the cached order and moves to 256
    assert m_old[16] == 768 and m_new[16] == 256
    m_old, _ = W.block_positions(W.LLAMA3_70B)
    assert m_old[1] - m_old[0] == 64
