"""The C ABI driven from plain C, with no torch in the process: the client in
tests/c/hkv_roundtrip.c takes device memory from hipMalloc and one stream from
hipStreamCreate.  It calls the put, the CRC, the fused put + CRC and the fetch
on inputs this test writes, and its outputs are checked against the CPU
oracle.

Bar, as in the other parity tests: records and CRCs bit-exact; values, and
keys of blocks with a zero delta, exact; other keys within 2e-6 * ||k|| (fp32
pages) or one unit in the last place (16-bit pages).  Records of skipped
blocks and pages no block maps to keep the bytes the client filled them with."""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest
import torch

import oracle as O
from parity_util import compare_fetch_block

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c", "hkv_roundtrip")
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
FMT_CODE = {"fp8": 0, "int4": 1}
PAIRS_CODE = {"interleaved": 0, "half_split": 1}

# name, layers, pages, tokens per block, heads, source dtype, format, pairs,
# page dtype, RoPE base, put table, fetch table
CASES = [
    ("fp8-tiny-f32", 1, 4, 16, 8, "f32", "fp8", "interleaved", "f32", 10000.0,
     [2, 0, 3, 1], [1, 3, 0, 2]),
    # 60 vectors per block: the fused call runs the put and then the CRC kernel
    ("int4-ragged-f16-bf16", 3, 5, 12, 5, "f16", "int4", "half_split", "bf16", 500000.0,
     [4, -1, 0, 2, 7, 1], [0, -1, 4, 1, -1, 9]),
    # 512 vectors per block: the one-pass fused put + CRC
    ("fp8-64x8-bf16-f16", 2, 6, 64, 8, "bf16", "fp8", "half_split", "f16", 1e6,
     [5, 3, 0, 4, 1, 2], [2, 0, 5, 3, 1, 4]),
]


def _as_source(x: np.ndarray, dtype: str):
    """(bytes in the source dtype, the float32 values the GPU reads)."""
    t = torch.from_numpy(x)
    if dtype == "f32":
        return x.astype(np.float32).tobytes(), x.astype(np.float32)
    td = torch.float16 if dtype == "f16" else torch.bfloat16
    c = t.to(td)
    return c.view(torch.int16).numpy().tobytes(), c.float().numpy()


def _read_pages(path: str, dtype: str, shape) -> np.ndarray:
    raw = np.fromfile(path, dtype=np.uint8)
    if dtype == "f32":
        return raw.view(np.float32).reshape(shape).astype(np.float64)
    bits = raw.view(np.uint16).reshape(shape)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_c_client_against_oracle(case, tmp_path):
    name, L, P, tb, H, src_dtype, fmt, pairs, dst_dtype, base, put_table, fetch_table = case
    if not os.path.exists(CLIENT):
        pytest.fail(f"{CLIENT} is not built; run `python -c \"import __graft_entry__ as g; "
                    "g.build()\"`")
    print(f"[c-abi] {name}", flush=True)
    nb = len(put_table)
    rng = np.random.default_rng([71, L, P, tb, H])
    kp = rng.standard_normal((L, P, tb, H, 128)).astype(np.float32)
    vp = (rng.standard_normal((L, P, tb, H, 128)) * 2.5).astype(np.float32)
    dm = rng.integers(-40000, 40000, size=nb).astype(np.int32)
    dm[1] = 0
    put_tab = np.array(put_table, dtype=np.int32)
    fetch_tab = np.array(fetch_table, dtype=np.int32)

    d = str(tmp_path)
    k_bytes, k_seen = _as_source(kp, src_dtype)
    v_bytes, v_seen = _as_source(vp, src_dtype)
    with open(os.path.join(d, "params.txt"), "w") as f:
        f.write(f"{L} {nb} {tb} {H} {P} {DTYPE_CODE[src_dtype]} {FMT_CODE[fmt]} "
                f"{PAIRS_CODE[pairs]} {DTYPE_CODE[dst_dtype]} {base!r}\n")
    for fname, data in (("k_src.bin", k_bytes), ("v_src.bin", v_bytes),
                        ("put_table.bin", put_tab.tobytes()),
                        ("fetch_table.bin", fetch_tab.tobytes()), ("delta.bin", dm.tobytes())):
        with open(os.path.join(d, fname), "wb") as f:
            f.write(data)

    r = subprocess.run([CLIENT, d], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"client exited {r.returncode}: {r.stderr}"

    ref, live = O.put(k_seen, v_seen, put_tab, fmt)
    rb = ref.shape[-1]
    got = np.fromfile(os.path.join(d, "records.bin"), dtype=np.uint8).reshape(L, nb, rb)
    fused = np.fromfile(os.path.join(d, "records_fused.bin"), dtype=np.uint8).reshape(L, nb, rb)
    for b in range(nb):
        if live[b]:
            assert np.array_equal(got[:, b], ref[:, b]), f"{name}: record {b} differs"
            assert np.array_equal(fused[:, b], ref[:, b]), f"{name}: fused record {b} differs"
        else:
            assert np.all(got[:, b] == 0xA5), f"{name}: skipped record {b} was written"
            assert np.all(fused[:, b] == 0xA5), f"{name}: skipped fused record {b} was written"

    # the CRC kernel covers every record, skipped ones with their fill bytes
    crc = np.fromfile(os.path.join(d, "crc.bin"), dtype=np.uint32).reshape(L, nb)
    assert np.array_equal(crc, O.crc32_records(got)), f"{name}: CRC differs from the oracle"
    crc_fused = np.fromfile(os.path.join(d, "crc_fused.bin"), dtype=np.uint32).reshape(L, nb)
    ref_crc = O.crc32_records(ref)
    assert np.array_equal(crc_fused[:, live], ref_crc[:, live]), f"{name}: fused CRC differs"

    kr, vd = O.fetch_exact(ref, fmt, tb, H, dm, base, pairs)
    kd, _ = O.dequant_records(ref, fmt, tb, H)
    shape = (L, P, tb, H, 128)
    kg = _read_pages(os.path.join(d, "k_out.bin"), dst_dtype, shape)
    vg = _read_pages(os.path.join(d, "v_out.bin"), dst_dtype, shape)
    written = set()
    for b, page in enumerate(fetch_tab):
        if page < 0 or page >= P:
            continue
        assert live[b], "the fetch tables list only blocks that were put"
        written.add(int(page))
        compare_fetch_block(kg[:, page], vg[:, page], kr[:, b], vd[:, b], kd[:, b], dst_dtype,
                            int(dm[b]), f"{name} block {b}")
    raw_k = np.fromfile(os.path.join(d, "k_out.bin"), dtype=np.uint8).reshape(L, P, -1)
    raw_v = np.fromfile(os.path.join(d, "v_out.bin"), dtype=np.uint8).reshape(L, P, -1)
    for p in range(P):
        if p not in written:
            assert np.all(raw_k[:, p] == 0xEE) and np.all(raw_v[:, p] == 0xEE), \
                f"{name}: page {p} was written"
