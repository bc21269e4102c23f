"""The put's quotient x / s at the rounding edges of the codes.

The put rounds the fp32 quotient x / s to an FP8 E4M3 code or to an INT4
integer, and the quotient must be the correctly rounded IEEE fp32 one (the
HyperCache post's FP8 and INT4 records; the oracle divides with numpy's IEEE
fp32 division).  The kernel forms it from a reciprocal and one correction
step, so the places where a quotient one fp32 ulp off would change a code --
quotients at or next to a midpoint between two codes -- are driven through
the put here for every fp16 scale value the put can store:

* every positive fp16 significand at the exponents -14, -8, -1, 0, 1, 7 and
  15, and every fp16 subnormal k * 2^-24;
* the two clamped scales: 2^-24 for an amax whose scale underflows fp16 and
  65504 for one whose scale overflows it.

Each vector's amax is qmax * s, so the stored scale is exactly s; the other
elements sit at m * s (exact in fp32) and at the fp32 numbers one and two
ulps either side of it, for every midpoint m between adjacent FP8 codes below
448 or every half-integer below 7 (INT4), and for the codes themselves, both
signs.  Records (codes and scales) must equal the oracle's byte for byte.

A second test sweeps the kernel's division routine itself against IEEE
division on the GPU: every fp32 significand of x against every fp16
significand of s (2^33 pairs), which by exact power-of-two scaling covers
every quotient the put forms in the normal range."""
from __future__ import annotations

import ctypes
import os

import numpy as np
import pytest
import torch

import oracle as O
from quantization_rope_reuse_amd import hkv

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
HERE = os.path.dirname(os.path.abspath(__file__))


def _e4m3_positive_values():
    """Values of the E4M3FN codes 0x00..0x7E from the format's definition
    (bias 7, 3 mantissa bits, subnormals m/8 * 2^-6)."""
    c = np.arange(127)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7))


def _scales():
    """Every fp16 scale value the test drives: subnormals and all
    significands at seven exponents."""
    sub = np.arange(1, 1024, dtype=np.float64) * 2.0 ** -24
    normal = [(1024 + np.arange(1024, dtype=np.float64)) * 2.0 ** (e - 10)
              for e in (-14, -8, -1, 0, 1, 7, 15)]
    return np.concatenate([sub] + normal)


def _neighbours(x32, n=2):
    """x and the fp32 numbers 1..n ulps either side of it."""
    out = [x32]
    up, down = x32.copy(), x32.copy()
    for _ in range(n):
        up = np.nextafter(up, np.float32(np.inf))
        down = np.nextafter(down, np.float32(-np.inf))
        out += [up, down]
    return np.stack(out, axis=-1)


def _vectors(scales, amax_of_s, targets):
    """Vectors of 128 fp32 elements per scale: element 0 is amax_of_s(s), the
    rest are targets * s with their neighbours and both signs, padded with
    zeros.  Returns (vectors [n, 128] float32, scale per vector)."""
    rows, svals = [], []
    for s in scales:
        base = (targets * s).astype(np.float32)            # exact: few significant bits
        assert np.all(base.astype(np.float64) == targets * s)
        vals = _neighbours(base).reshape(-1)
        vals = np.concatenate([vals, -vals])
        amax = np.float32(amax_of_s(s))
        assert np.all(np.abs(vals) <= amax)
        per = 127
        n = -(-vals.size // per)
        block = np.zeros((n, 128), np.float32)
        block[:, 0] = amax
        flat = np.zeros(n * per, np.float32)
        flat[:vals.size] = vals
        block[:, 1:] = flat.reshape(n, per)
        rows.append(block)
        svals += [s] * n
    return np.concatenate(rows), np.array(svals)


def _run_put(x, fmt):
    """Put of the vectors x [n, 128] (fp32 source) as K and V of one layer of
    blocks of 16 tokens x 8 heads; returns GPU records and the oracle's."""
    per_block = 2 * 128
    n = -(-x.shape[0] // per_block) * per_block
    xs = np.zeros((n, 128), np.float32)
    xs[:x.shape[0]] = x
    nb = n // per_block
    k = xs[0::2].reshape(1, nb, 16, 8, 128)
    v = xs[1::2].reshape(1, nb, 16, 8, 128)
    table = np.arange(nb, dtype=np.int32)
    rec = hkv.alloc_records(1, nb, fmt, 16, 8, device=DEV)
    rec.fill_(0xA5)
    put = hkv.quant_fp8 if fmt == "fp8" else hkv.quant_int4
    put(torch.from_numpy(k).to(DEV), torch.from_numpy(v).to(DEV),
        torch.from_numpy(table).to(DEV), rec)
    torch.cuda.synchronize()
    ref, _ = O.put(k, v, table, fmt)
    return rec.cpu().numpy(), ref, nb


def _stored_scales(rec, fmt, nb):
    kc, vc, ks, vs = O.split_records(rec, fmt, 16, 8)
    out = np.empty((nb * 256,), np.float64)
    out[0::2] = ks.reshape(-1)
    out[1::2] = vs.reshape(-1)
    return out


def _check(x, svals, fmt, what):
    got, ref, nb = _run_put(x, fmt)
    # the construction gives the intended scale (else the test tests nothing)
    stored = _stored_scales(ref, fmt, nb)[:x.shape[0]]
    assert np.array_equal(stored, svals), f"{what}: the oracle stored other scales"
    bad = got != ref
    assert not bad.any(), (f"{what}: {int(bad.sum())} record bytes differ from the oracle "
                           f"(first at byte {np.argwhere(bad)[0].tolist()})")


@pytest.mark.parametrize("fmt", ["fp8", "int4"])
def test_quotient_at_code_midpoints_every_scale(fmt):
    print(f"[division] {fmt} midpoints", flush=True)
    if fmt == "fp8":
        codes = _e4m3_positive_values()                   # 0 .. 448
        mids = (codes[:-1] + codes[1:]) / 2
        targets = np.concatenate([mids, codes[1:-1]])
        qmax = 448.0
    else:
        targets = np.concatenate([np.arange(7) + 0.5, np.arange(1, 7, dtype=np.float64)])
        qmax = 7.0
    x, svals = _vectors(_scales(), lambda s: qmax * s, targets)
    _check(x, svals, fmt, f"{fmt}, all fp16 scales")


@pytest.mark.parametrize("fmt", ["fp8", "int4"])
def test_quotient_at_code_midpoints_clamped_scales(fmt):
    """The clamped scales.  Underflow: amax = qmax * 2^-25 makes amax / qmax
    exactly half the smallest fp16 subnormal, a tie that rounds to zero, so
    the stored scale is the clamp 2^-24.  Overflow: amax = qmax * 65520 makes
    the scale round past 65504 to infinity, so it is clamped to 65504 and
    the amax element itself saturates."""
    print(f"[division] {fmt} clamped scales", flush=True)
    if fmt == "fp8":
        codes = _e4m3_positive_values()
        mids = (codes[:-1] + codes[1:]) / 2
        targets = np.concatenate([mids, codes[1:-1]])
        qmax = 448.0
    else:
        targets = np.concatenate([np.arange(7) + 0.5, np.arange(1, 7, dtype=np.float64)])
        qmax = 7.0
    lo_t = targets[targets * 2.0 ** -24 < qmax * 2.0 ** -25]     # neighbours stay below amax
    x_lo, s_lo = _vectors([2.0 ** -24], lambda s: qmax * 2.0 ** -25, lo_t)
    x_hi, s_hi = _vectors([65504.0], lambda s: qmax * 65520.0, targets)
    _check(np.concatenate([x_lo, x_hi]), np.concatenate([s_lo, s_hi]), fmt,
           f"{fmt}, clamped scales")


# ---------------------------------------------------------------------------
# The division routine against IEEE division, exhaustively per binade
# ---------------------------------------------------------------------------

def _sweep_lib():
    path = os.path.join(HERE, "hip", "libdiv_sweep.so")
    if not os.path.exists(path):
        pytest.fail(f"{path} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    lib.div_sweep.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.div_sweep.restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("x_exp,s_exp", [(0, 0), (0, -24), (-30, 15), (20, -10), (-20, 0)])
def test_division_routine_exhaustive(x_exp, s_exp):
    """Every x = (1 + i / 2^23) * 2^x_exp against every s = (1 + j / 2^10) *
    2^s_exp: the put's division routine (reciprocal and one correction step)
    equals the correctly rounded fp32 quotient bit for bit."""
    print(f"[division] sweep 2^{x_exp} / 2^{s_exp}", flush=True)
    lib = _sweep_lib()
    out = torch.zeros(2, dtype=torch.int64, device=DEV)
    out[1] = -1
    st = lib.div_sweep(x_exp, s_exp, ctypes.c_void_p(out.data_ptr()),
                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, f"launch status {st}"
    torch.cuda.synchronize()
    n_bad, first = (int(v) for v in out.cpu())
    assert n_bad == 0, (f"{n_bad} of 2^33 quotients differ; first x significand "
                        f"{first >> 10:#x}, s significand {first & 1023:#x}")
