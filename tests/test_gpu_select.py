"""GPU parity of the recompute selection (per-token layer-0 drift, then the
top 15%) through the C ABI, against the CPU oracle.

Bar.  Drift: |gpu - exact| <= (m + 10) * 2^-24 * exact, with m the number of
terms one lane sums (fp32 differences, squares and sums; derivation next to
the tolerance below), and exactly 0 where the two rows are equal.
Selection: bit-exact against the oracle's selection applied to the GPU's own
drift values (the decision is taken in fp32 on both sides); against the
float64 drift, the two selections may differ only among tokens whose exact
drift lies within the drift tolerance of the k-th value."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle as O
from parity_util import TORCH_OF, host_f64
from quantization_rope_reuse_amd import hkv
from quantization_rope_reuse_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U = 2.0 ** -24


def drift_rel_tol(d_model: int, dtype: str) -> float:
    """One lane sums m = e * ceil(d / (64 e)) + 1 squares (e elements per
    16-byte load, plus one tail element); the 64 lane sums meet in a 6-level
    tree.  Each difference and each fma rounds once (relative 2u on a
    square), the sums of non-negative terms add at most (m + 6) u, and the
    square root halves that and rounds once more: (m + 10) u covers it."""
    e = 4 if dtype == "f32" else 8
    m = e * -(-d_model // (64 * e)) + 1
    return (m + 10) * U


def check_drift(gpu: np.ndarray, exact: np.ndarray, d_model: int, dtype: str, what: str):
    tol = drift_rel_tol(d_model, dtype)
    zero = exact == 0
    assert np.all(gpu[zero] == 0), f"{what}: equal rows must give 0"
    rel = np.abs(gpu[~zero] - exact[~zero]) / exact[~zero]
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= tol, f"{what}: drift relative error {worst:.3e} > {tol:.3e}"
    return worst


def check_selection_against_exact(sel: np.ndarray, exact: np.ndarray, k: int, rel_tol: float):
    """The GPU's set may differ from the exact-drift selection only near the
    k-th exact value."""
    want = O.select_top_tokens(exact, k)
    if k == 0:
        return
    kth = np.sort(exact)[::-1][k - 1]
    band = rel_tol * kth * 2
    diff = np.setxor1d(sel, want)
    assert np.all(np.abs(exact[diff] - kth) <= band), "selection differs away from the threshold"


def _dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV, TORCH_OF[dtype])


def test_gqa_prefix_drift_and_selection():
    w = W.DRIFT_GQA
    print(f"[select] {w.name}", flush=True)
    c, f = W.host_hidden_states(w)
    drift = hkv.token_drift(_dev(c, w.dtype), _dev(f, w.dtype))
    k = O.recompute_count(w.n_tokens)
    sel = hkv.select_top_tokens(drift, k)
    torch.cuda.synchronize()
    dg = drift.cpu().numpy()
    exact = O.token_drift(c, f)
    check_drift(dg, exact, w.d_model, w.dtype, w.name)
    assert k == 192
    s = sel.cpu().numpy()
    assert np.array_equal(s, O.select_top_tokens(dg, k))
    check_selection_against_exact(s, exact, k, drift_rel_tol(w.d_model, w.dtype))
    # the unmoved lead chunk has zero drift and is never selected
    assert not dg[:w.lead_tokens].any() and s.min() >= w.lead_tokens


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d_model,pad", [(4096, 0), (1000, 24), (100, 28), (3, 5), (1, 7), (0, 8),
                                         (520, 8)])
def test_drift_widths_strides_dtypes(dtype, d_model, pad):
    rng = np.random.default_rng(d_model * 7 + pad)
    n = 77                                           # not a multiple of 4 tokens per group
    width = d_model + pad                            # row stride, 16-byte multiple for all dtypes
    big_c = rng.standard_normal((n, width)).astype(np.float32)
    big_f = big_c + rng.standard_normal((n, width)).astype(np.float32) * \
        rng.uniform(0.0, 0.5, (n, 1)).astype(np.float32)
    big_f[5] = big_c[5]                              # one equal row
    tc = _dev(big_c, dtype)
    tf = _dev(big_f, dtype)
    a, b = tc[:, :d_model], tf[:, :d_model]
    print(f"[select] drift {dtype} d={d_model} stride={width}", flush=True)
    drift = hkv.token_drift(a, b)
    torch.cuda.synchronize()
    exact = O.token_drift(host_f64(a), host_f64(b))
    check_drift(drift.cpu().numpy(), exact, d_model, dtype, f"{dtype} d={d_model}")


def test_drift_extreme_values():
    # large and tiny magnitudes: fp32 squares stay in range for fp16/bf16 data
    n, d = 8, 512
    c = np.zeros((n, d), np.float32)
    f = np.zeros((n, d), np.float32)
    f[0, :] = 60000.0                                # fp16 near its maximum
    f[1, 0] = 6e-8                                   # fp16 subnormal
    f[2, ::2] = 1e-3
    c[3, :] = -1e4
    f[3, :] = 1e4
    f[4, 7] = -2.0
    for dtype in ("f16", "bf16", "f32"):
        a, b = _dev(c, dtype), _dev(f, dtype)
        drift = hkv.token_drift(a, b).cpu().numpy()
        exact = O.token_drift(host_f64(a), host_f64(b))
        check_drift(drift, exact, d, dtype, f"extremes {dtype}")
        assert drift[4] == 2.0 and drift[5] == 0.0


SELECT_CASES = [
    ("all equal", np.full(3000, 2.5, np.float32), 450),
    ("nan inf and signed zeros",
     np.array([0.0, -0.0, np.nan, 1.0, np.inf, -np.inf, -0.0, 0.0, np.nan, -1.0] * 150,
              np.float32), 700),
    ("negatives", -np.abs(np.random.default_rng(3).standard_normal(2049)).astype(np.float32), 300),
    ("k equals n", np.random.default_rng(4).standard_normal(1500).astype(np.float32), 1500),
    ("k one", np.random.default_rng(5).standard_normal(1025).astype(np.float32), 1),
    ("single token", np.array([0.5], np.float32), 1),
    ("subnormals", (np.random.default_rng(6).integers(1, 50, 4000) * 1e-45).astype(np.float32),
     600),
    ("ties across tiles", np.repeat(np.arange(40, dtype=np.float32), 97), 1000),
    ("one bit apart",
     (np.float32(1.0) + np.random.default_rng(7).integers(0, 3, 5000).astype(np.float32)
      * np.float32(2.0 ** -23)), 777),
]


PATHS = [True, None]                     # many workgroups with a workspace; one workgroup


@pytest.mark.parametrize("ws", PATHS, ids=["workspace", "one_group"])
@pytest.mark.parametrize("name,values,k", SELECT_CASES, ids=[c[0] for c in SELECT_CASES])
def test_selection_edge_cases(name, values, k, ws):
    print(f"[select] {name} n={values.size} k={k} workspace={ws}", flush=True)
    d = torch.from_numpy(values).to(DEV)
    sel = hkv.select_top_tokens(d, k, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), O.select_top_tokens(values, k)), name


@pytest.mark.parametrize("ws", PATHS, ids=["workspace", "one_group"])
def test_selection_large_random_and_empty(ws):
    rng = np.random.default_rng(8)
    n = 300_000
    v = (np.abs(rng.standard_normal(n)) * 4).astype(np.float16).astype(np.float32)  # many ties
    d = torch.from_numpy(v).to(DEV)
    for k in (1, 45_000, n - 1):
        print(f"[select] large n={n} k={k} workspace={ws}", flush=True)
        sel = hkv.select_top_tokens(d, k, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(sel.cpu().numpy(), O.select_top_tokens(v, k))
    out = torch.full((4,), -7, dtype=torch.int32, device=DEV)
    hkv.select_top_tokens(d, 0, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [-7] * 4             # k = 0 writes nothing


def test_selection_workspace_reused_across_sizes():
    # one workspace sized for the largest call serves smaller ones after it,
    # across the slice-size change at 65,536 tokens and ragged last slices
    rng = np.random.default_rng(9)
    ws = torch.empty(hkv.select_workspace_bytes(200_003), dtype=torch.uint8, device=DEV)
    for n in (200_003, 65_537, 65_536, 4_097, 4_096, 1_000, 1):
        v = rng.standard_normal(n).astype(np.float32)
        v[rng.integers(0, n, n // 10)] = 0.5                # ties
        k = max(1, (n * 15) // 100)
        print(f"[select] reused workspace n={n} k={k}", flush=True)
        sel = hkv.select_top_tokens(torch.from_numpy(v).to(DEV), k, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(sel.cpu().numpy(), O.select_top_tokens(v, k)), n


def test_side_stream_selection_matches():
    w = W.DRIFT_GQA
    c, f = W.host_hidden_states(w)
    a, b = _dev(c, w.dtype), _dev(f, w.dtype)
    k = O.recompute_count(w.n_tokens)
    base = hkv.select_top_tokens(hkv.token_drift(a, b), k)
    side = torch.cuda.Stream()
    ready = torch.cuda.Event()
    ready.record(torch.cuda.current_stream())
    side.wait_event(ready)
    with torch.cuda.stream(side):
        drift = torch.empty(w.n_tokens, dtype=torch.float32, device=DEV)
        sel = torch.empty(k, dtype=torch.int32, device=DEV)
    hkv.token_drift(a, b, out=drift, stream=side)
    hkv.select_top_tokens(drift, k, out=sel, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(sel, base)


@pytest.mark.parametrize("w", [W.DRIFT_QWEN3_8B, W.DRIFT_LLAMA3_70B], ids=lambda w: w.name)
def test_full_size_drift_and_selection(w):
    print(f"[select] full {w.name}", flush=True)
    c, f = W.device_hidden_states(w, DEV)
    drift = hkv.token_drift(c, f)
    k = O.recompute_count(w.n_tokens)
    sel = hkv.select_top_tokens(drift, k)
    sel1 = hkv.select_top_tokens(drift, k, workspace=None)
    torch.cuda.synchronize()
    dg = drift.cpu().numpy()
    s = sel.cpu().numpy()
    assert np.array_equal(s, O.select_top_tokens(dg, k))
    assert np.array_equal(sel1.cpu().numpy(), s)
    assert not dg[:w.lead_tokens].any() and (dg[w.lead_tokens:] > 0).all()
    rng = np.random.default_rng(90)
    starts = w.lead_tokens + w.chunk_tokens * np.arange(w.n_chunks)
    rows = np.unique(np.concatenate([[0, w.lead_tokens - 1, w.n_tokens - 1], starts[:8],
                                     s[:16], rng.integers(0, w.n_tokens, 40)]))
    idx = torch.from_numpy(rows).to(DEV)
    exact = O.token_drift(host_f64(c[idx]), host_f64(f[idx]))
    check_drift(dg[rows], exact, w.d_model, w.dtype, w.name)
    # the drift recipe peaks right after chunk boundaries: the first quarter
    # of each chunk holds well over a quarter of the selected tokens
    j = (s - w.lead_tokens) % w.chunk_tokens
    assert np.mean(j < w.chunk_tokens // 4) > 0.375
    del c, f
    torch.cuda.empty_cache()
    assert math.isfinite(float(dg.max()))
