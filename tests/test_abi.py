"""The C-ABI library: it loads, exports every function include/hkv.h
declares, and rejects bad arguments on the host before any HIP call (these
tests run without a GPU)."""
import ctypes

import pytest

from quantization_rope_reuse_amd import hkv

H = hkv


def test_exports_every_declared_symbol():
    names = H.declared_symbols()
    assert set(names) == {"hkv_quant_fp8", "hkv_quant_int4", "hkv_fetch_dequant_rope_shift",
                          "hkv_crc32_blocks", "hkv_record_bytes", "hkv_status_string",
                          "hkv_page_visit_order", "hkv_fetch_dequant_rope_shift_tokens",
                          "hkv_stream_pair_create", "hkv_stream_destroy", "hkv_token_drift",
                          "hkv_select_top_tokens", "hkv_frame_headers", "hkv_frame_verify",
                          "hkv_frame_delta_m", "hkv_select_workspace_bytes",
                          "hkv_quant_fp8_crc", "hkv_quant_int4_crc",
                          "hkv_quant_crc_workspace_bytes", "hkv_stream_probe",
                          "hkv_stream_probe_put", "hkv_quant_fp8_crc_noalloc",
                          "hkv_fetch_staged"}
    lib = H.lib()
    for n in names:
        assert getattr(lib, n) is not None


def test_header_is_plain_c(tmp_path):
    """include/hkv.h compiles as C99 with every warning an error, and a C
    program that takes the address of every declared function links against
    libhkv.so and runs a host-only call."""
    import os
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs gcc and the ROCm headers")
    names = H.declared_symbols()
    src = tmp_path / "uses_hkv.c"
    src.write_text('#include "hkv.h"\n'
                   "int main(void) {\n"
                   + "".join(f"  (void)&{n};\n" for n in names)
                   + "  return hkv_record_bytes(HKV_FP8_E4M3, 64, 8, HKV_HEAD_DIM) == 133120 &&\n"
                     "         hkv_status_string(HKV_ERR_UNSUPPORTED) != 0 ? 0 : 1;\n}\n")
    pkg = os.path.dirname(H.LIB_PATH)
    include = os.path.join(os.path.dirname(pkg), "include")
    exe = tmp_path / "uses_hkv"
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I", "/opt/rocm/include", "-I", include, str(src), "-o", str(exe),
                        "-L", pkg, "-lhkv", f"-Wl,-rpath,{pkg}"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert subprocess.run([str(exe)], timeout=60).returncode == 0


def test_record_bytes():
    assert H.record_bytes("fp8", 64, 8) == 133120
    assert H.record_bytes("int4", 64, 8) == 67584
    assert H.record_bytes("fp8", 16, 8) == 33280
    assert H.record_bytes("int4", 1, 1) == 132
    assert H.lib().hkv_record_bytes(7, 16, 8, 128) == -1
    assert H.lib().hkv_record_bytes(0, 16, 8, 64) == -1
    assert H.lib().hkv_record_bytes(0, 0, 8, 128) == -1


def test_status_strings():
    assert H.status_string(0) == "ok"
    assert H.status_string(-1) == "invalid argument"
    assert H.status_string(-2) == "unsupported request"
    assert H.status_string(-3) == "HIP launch error"
    assert H.status_string(5) == "unknown status"


FAKE = 0x7F0000000000          # a 16-byte aligned address never dereferenced


def _shape(**kw):
    d = dict(n_layers=2, n_blocks=4, block_tokens=16, n_kv_heads=8, head_dim=128)
    d.update(kw)
    return H.Shape(**d)


def _pages(**kw):
    d = dict(k=FAKE, v=FAKE + 4096, layer_stride=4 * 16 * 8 * 128, page_stride=16 * 8 * 128,
             token_stride=8 * 128, head_stride=128, num_pages=4)
    d.update(kw)
    return H.Pages(**d)


def _recs(**kw):
    d = dict(base=FAKE, layer_stride_bytes=4 * 33280, block_stride_bytes=33280)
    d.update(kw)
    return H.Records(**d)


def _quant(shape, pages, dtype, table, recs):
    return H.lib().hkv_quant_fp8(ctypes.byref(shape) if shape is not None else None,
                                 ctypes.byref(pages) if pages is not None else None, dtype,
                                 ctypes.c_void_p(table),
                                 ctypes.byref(recs) if recs is not None else None, None)


def _fetch(shape, recs, table, dm, base, pairs, pages, dtype, fmt=0):
    return H.lib().hkv_fetch_dequant_rope_shift(
        ctypes.byref(shape), fmt, ctypes.byref(recs), ctypes.c_void_p(table),
        ctypes.c_void_p(dm), None, base, pairs, ctypes.byref(pages), dtype, None)


BAD_QUANT = [
    ("null shape", lambda: _quant(None, _pages(), 0, FAKE, _recs())),
    ("null pages", lambda: _quant(_shape(), None, 0, FAKE, _recs())),
    ("null records", lambda: _quant(_shape(), _pages(), 0, FAKE, None)),
    ("null table", lambda: _quant(_shape(), _pages(), 0, 0, _recs())),
    ("head_dim 64", lambda: _quant(_shape(head_dim=64), _pages(), 0, FAKE, _recs())),
    ("zero heads", lambda: _quant(_shape(n_kv_heads=0), _pages(), 0, FAKE, _recs())),
    ("zero block tokens", lambda: _quant(_shape(block_tokens=0), _pages(), 0, FAKE, _recs())),
    ("negative layers", lambda: _quant(_shape(n_layers=-1), _pages(), 0, FAKE, _recs())),
    ("bad dtype", lambda: _quant(_shape(), _pages(), 3, FAKE, _recs())),
    ("misaligned k", lambda: _quant(_shape(), _pages(k=FAKE + 8), 0, FAKE, _recs())),
    ("null v", lambda: _quant(_shape(), _pages(v=0), 0, FAKE, _recs())),
    ("odd head stride", lambda: _quant(_shape(), _pages(head_stride=130), 2, FAKE, _recs())),
    ("negative stride", lambda: _quant(_shape(), _pages(page_stride=-128), 0, FAKE, _recs())),
    ("negative num_pages", lambda: _quant(_shape(), _pages(num_pages=-1), 0, FAKE, _recs())),
    ("misaligned records", lambda: _quant(_shape(), _pages(), 0, FAKE, _recs(base=FAKE + 4))),
    ("short block stride", lambda: _quant(_shape(), _pages(), 0, FAKE,
                                          _recs(block_stride_bytes=33264))),
    ("unaligned block stride", lambda: _quant(_shape(), _pages(), 0, FAKE,
                                              _recs(block_stride_bytes=33288))),
]


@pytest.mark.parametrize("name,call", BAD_QUANT, ids=[b[0] for b in BAD_QUANT])
def test_quant_rejects_bad_arguments(name, call):
    assert call() == H.ERR_INVALID_ARG


def test_unsupported_sizes():
    assert _quant(_shape(n_layers=70000), _pages(), 0, FAKE, _recs()) == H.ERR_UNSUPPORTED


def test_empty_calls_launch_nothing():
    assert _quant(_shape(n_layers=0), _pages(), 0, FAKE, _recs()) == H.OK
    assert _quant(_shape(n_blocks=0), _pages(), 0, 0, _recs()) == H.OK
    s = _shape(n_blocks=0)
    assert _fetch(s, _recs(), 0, 0, 1e4, 0, _pages(), 0) == H.OK


BAD_FETCH = [
    ("zero base", dict(base=0.0)),
    ("negative base", dict(base=-10000.0)),
    ("nan base", dict(base=float("nan"))),
    ("inf base", dict(base=float("inf"))),
    ("bad pairs", dict(pairs=2)),
    ("bad format", dict(fmt=2)),
    ("bad dtype", dict(dtype=-1)),
    ("null delta", dict(dm=0)),
    ("null table", dict(table=0)),
]


@pytest.mark.parametrize("name,kw", BAD_FETCH, ids=[b[0] for b in BAD_FETCH])
def test_fetch_rejects_bad_arguments(name, kw):
    a = dict(table=FAKE, dm=FAKE, base=1e4, pairs=0, dtype=0, fmt=0)
    a.update(kw)
    st = _fetch(_shape(), _recs(), a["table"], a["dm"], a["base"], a["pairs"], _pages(),
                a["dtype"], a["fmt"])
    assert st == H.ERR_INVALID_ARG


def test_fetch_tokens_rejects_bad_arguments():
    lib = H.lib()
    s, r, p = _shape(), _recs(), _pages()
    call = lambda **kw: lib.hkv_fetch_dequant_rope_shift_tokens(
        ctypes.byref(s), kw.get("fmt", 0), ctypes.byref(r), ctypes.c_void_p(kw.get("t", FAKE)),
        ctypes.c_void_p(kw.get("dm", FAKE)), None, kw.get("base", 1e4), kw.get("pairs", 0),
        ctypes.byref(p), kw.get("dt", 0), None)
    assert call(dm=0) == H.ERR_INVALID_ARG
    assert call(t=0) == H.ERR_INVALID_ARG
    assert call(base=-1.0) == H.ERR_INVALID_ARG
    assert call(pairs=5) == H.ERR_INVALID_ARG
    assert call(fmt=3) == H.ERR_INVALID_ARG


def test_stream_helpers_reject_null_arguments():
    lib = H.lib()
    p = ctypes.c_void_p()
    assert lib.hkv_stream_pair_create(8, None, ctypes.byref(p)) == H.ERR_INVALID_ARG
    assert lib.hkv_stream_pair_create(8, ctypes.byref(p), None) == H.ERR_INVALID_ARG
    assert lib.hkv_stream_destroy(None) == H.ERR_INVALID_ARG


def test_crc_rejects_bad_arguments():
    lib = H.lib()
    s, r = _shape(), _recs()
    assert lib.hkv_crc32_blocks(ctypes.byref(s), 0, ctypes.byref(r), None, None) == H.ERR_INVALID_ARG
    assert lib.hkv_crc32_blocks(ctypes.byref(s), 9, ctypes.byref(r), ctypes.c_void_p(FAKE),
                                None) == H.ERR_INVALID_ARG
    r2 = _recs(base=0)
    assert lib.hkv_crc32_blocks(ctypes.byref(s), 0, ctypes.byref(r2), ctypes.c_void_p(FAKE),
                                None) == H.ERR_INVALID_ARG


def test_page_order_rejects_bad_arguments():
    lib = H.lib()
    assert lib.hkv_page_visit_order(None, 4, 4, ctypes.c_void_p(FAKE), None) == H.ERR_INVALID_ARG
    assert lib.hkv_page_visit_order(ctypes.c_void_p(FAKE), 4, 4, None, None) == H.ERR_INVALID_ARG
    assert lib.hkv_page_visit_order(ctypes.c_void_p(FAKE), -1, 4, ctypes.c_void_p(FAKE),
                                    None) == H.ERR_INVALID_ARG
    assert lib.hkv_page_visit_order(None, 0, 4, None, None) == H.OK
    # the O(n^2) rank kernel takes at most 65,536 blocks
    assert lib.hkv_page_visit_order(ctypes.c_void_p(FAKE), (1 << 16) + 1, 4,
                                    ctypes.c_void_p(FAKE), None) == H.ERR_UNSUPPORTED


def test_binding_validates_tensors_before_calling():
    import torch
    k = torch.zeros((4, 16, 8, 128), dtype=torch.float16)
    with pytest.raises(ValueError):
        H.quant_fp8(k, k.float(), torch.zeros(4, dtype=torch.int32),
                    torch.zeros((1, 4, 33280), dtype=torch.uint8))
    with pytest.raises(ValueError):
        H.quant_fp8(k, k, torch.zeros(4, dtype=torch.int64),
                    torch.zeros((1, 4, 33280), dtype=torch.uint8))


def _drift(a=FAKE, b=FAKE + 4096, n=4, d=4096, stride=4096, dt=2, out=FAKE + 8192):
    return H.lib().hkv_token_drift(ctypes.c_void_p(a), ctypes.c_void_p(b), n, d, stride, dt,
                                   ctypes.c_void_p(out), None)


BAD_DRIFT = [
    ("bad dtype", dict(dt=3)),
    ("negative tokens", dict(n=-1)),
    ("negative width", dict(d=-8)),
    ("null cached", dict(a=0)),
    ("null fresh", dict(b=0)),
    ("null out", dict(out=0)),
    ("misaligned cached", dict(a=FAKE + 8)),
    ("misaligned out", dict(out=FAKE + 2)),
    ("row stride not 16 bytes", dict(stride=4100)),
    ("row stride below width", dict(stride=2048)),
    ("negative stride", dict(stride=-4096)),
]


@pytest.mark.parametrize("name,kw", BAD_DRIFT, ids=[b[0] for b in BAD_DRIFT])
def test_drift_rejects_bad_arguments(name, kw):
    assert _drift(**kw) == H.ERR_INVALID_ARG


def test_select_rejects_bad_arguments():
    lib = H.lib()
    call = lambda d=FAKE, n=100, k=15, o=FAKE + 4096, ws=None, wsb=0: lib.hkv_select_top_tokens(
        ctypes.c_void_p(d), n, k, ctypes.c_void_p(o), ctypes.c_void_p(ws), wsb, None)
    assert call(k=101) == H.ERR_INVALID_ARG
    assert call(k=-1) == H.ERR_INVALID_ARG
    assert call(n=-1, k=0) == H.ERR_INVALID_ARG
    assert call(d=0) == H.ERR_INVALID_ARG
    assert call(o=0) == H.ERR_INVALID_ARG
    assert call(d=FAKE + 2) == H.ERR_INVALID_ARG
    assert call(k=0, d=0, o=0) == H.OK               # empty: nothing launched
    need = H.select_workspace_bytes(100)
    assert call(ws=FAKE + 8192, wsb=need - 4) == H.ERR_INVALID_ARG      # too small
    assert call(ws=FAKE + 8200, wsb=need) == H.ERR_INVALID_ARG          # misaligned
    assert call(n=(1 << 30) + 1, k=1) == H.ERR_UNSUPPORTED
    assert _drift(n=0, a=0, b=0, out=0) == H.OK
    # one row: the stride is not used; zero width: the rows are not read
    assert _drift(n=1, stride=0, a=0) == H.ERR_INVALID_ARG
    assert _drift(n=3, d=0, stride=0, a=0, b=0, out=0) == H.ERR_INVALID_ARG


def test_selection_binding_validates_tensors():
    import torch
    with pytest.raises(ValueError):
        H.select_top_tokens(torch.zeros(8, dtype=torch.float64), 2)
    with pytest.raises(ValueError):
        H.token_drift(torch.zeros((4, 8)), torch.zeros((4, 8), dtype=torch.float16))
    with pytest.raises(ValueError):
        H.token_drift(torch.zeros((4, 8)), torch.zeros((4, 9)))


def _frames_view(**kw):
    d = dict(base=FAKE, layer_stride_bytes=4 * 33344, block_stride_bytes=33344)
    d.update(kw)
    return H.Records(**d)


def test_frame_calls_reject_bad_arguments():
    lib = H.lib()
    s = _shape()                                       # 16 tokens x 8 heads: 33,280 B records
    hdr = lambda fr, crc=FAKE, m=FAKE, lb=0, fmt=0, sh=s: lib.hkv_frame_headers(
        ctypes.byref(sh), fmt, ctypes.byref(fr), ctypes.c_void_p(crc), ctypes.c_void_p(m), lb,
        None)
    # a frame stride that cannot hold header + record
    assert hdr(_frames_view(block_stride_bytes=33280)) == H.ERR_INVALID_ARG
    assert hdr(_frames_view(layer_stride_bytes=33280, block_stride_bytes=33344)) == \
        H.ERR_INVALID_ARG
    assert hdr(_frames_view(base=FAKE + 8)) == H.ERR_INVALID_ARG
    assert hdr(_frames_view(block_stride_bytes=33352)) == H.ERR_INVALID_ARG   # not 16-B
    assert hdr(_frames_view(), crc=0) == H.ERR_INVALID_ARG
    assert hdr(_frames_view(), m=0) == H.ERR_INVALID_ARG
    assert hdr(_frames_view(), lb=-1) == H.ERR_INVALID_ARG
    assert hdr(_frames_view(), fmt=5) == H.ERR_INVALID_ARG
    assert hdr(_frames_view(), sh=_shape(block_tokens=70000, n_kv_heads=1)) == \
        H.ERR_UNSUPPORTED
    assert hdr(_frames_view(), sh=_shape(n_blocks=0), crc=0, m=0) == H.OK
    ver = lambda fr, out=FAKE, lb=0: lib.hkv_frame_verify(
        ctypes.byref(s), 0, ctypes.byref(fr), lb, ctypes.c_void_p(out), None)
    assert ver(_frames_view(), out=0) == H.ERR_INVALID_ARG
    assert ver(_frames_view(), lb=-3) == H.ERR_INVALID_ARG
    assert ver(_frames_view(block_stride_bytes=16)) == H.ERR_INVALID_ARG
    dl = lambda fr, m=FAKE, out=FAKE: lib.hkv_frame_delta_m(
        ctypes.byref(s), 0, ctypes.byref(fr), ctypes.c_void_p(m), ctypes.c_void_p(out), None)
    assert dl(_frames_view(), m=0) == H.ERR_INVALID_ARG
    assert dl(_frames_view(), out=0) == H.ERR_INVALID_ARG
    assert dl(_frames_view(base=0)) == H.ERR_INVALID_ARG


def test_frame_allocation_shapes():
    import torch
    fr = H.alloc_frames(2, 3, "fp8", 16, 8, device="cpu")
    assert fr.shape == (2, 3, 64 + 33280) and fr.stride(1) == 33408 and fr.stride(0) == 3 * 33408
    rec = H.frame_records(fr)
    assert rec.shape == (2, 3, 33280) and rec.data_ptr() == fr.data_ptr() + 64
    assert rec.data_ptr() % 128 == 0 and fr.data_ptr() % 128 == 64
    fr4 = H.alloc_frames(1, 2, "int4", 1, 1, device="cpu")
    assert fr4.shape[2] == 64 + 132 and fr4.stride(1) == 256
    assert fr.dtype == torch.uint8


def test_select_workspace_sizes():
    ws = H.select_workspace_bytes
    assert ws(-1) == -1 and ws((1 << 30) + 1) == -1
    assert ws(0) == 4 * 8
    assert ws(1) == 4 * (1 * (3 * 2048 + 2) + 8)
    assert ws(65536) == 4 * (16 * (3 * 2048 + 2) + 8)
    assert ws(65537) == 4 * (33 * (3 * 2048 + 2) + 8)      # 33 slices of 2,048 tokens
    assert ws(1 << 30) == 4 * (64 * (3 * 2048 + 2) + 8)


def test_fused_put_crc_rejects_bad_arguments():
    lib = H.lib()
    s, p, r = _shape(), _pages(), _recs()           # 16 x 8 = 128 vectors: fused path
    need = lib.hkv_quant_crc_workspace_bytes(ctypes.byref(s), 0)
    assert need == 2 * 4 * (33280 // 128) * 4
    assert lib.hkv_quant_crc_workspace_bytes(ctypes.byref(_shape(head_dim=64)), 0) == -1
    assert lib.hkv_quant_crc_workspace_bytes(ctypes.byref(s), 9) == -1
    # 5 x 3 = 15 vectors: no workspace (put, then the CRC kernel)
    assert lib.hkv_quant_crc_workspace_bytes(ctypes.byref(_shape(block_tokens=5, n_kv_heads=3)),
                                             1) == 0
    call = lambda crc=FAKE, ws=FAKE + 4096, wsb=need, sh=s: lib.hkv_quant_fp8_crc(
        ctypes.byref(sh), ctypes.byref(p), 0, ctypes.c_void_p(FAKE), ctypes.byref(r),
        ctypes.c_void_p(crc), ctypes.c_void_p(ws), wsb, None, None)
    assert call(crc=0) == H.ERR_INVALID_ARG
    assert call(ws=0) == H.ERR_INVALID_ARG
    assert call(wsb=need - 1) == H.ERR_INVALID_ARG
    assert call(ws=FAKE + 4100) == H.ERR_INVALID_ARG               # misaligned
    assert call(sh=_shape(n_blocks=0), crc=0, ws=0, wsb=0) == H.OK


def test_noalloc_put_crc_rejects_bad_arguments_and_oversized_shapes():
    """hkv_quant_fp8_crc_noalloc checks its arguments like hkv_quant_fp8_crc
    and refuses, before any HIP call, a shape whose scratch need exceeds
    HKV_NOALLOC_SCRATCH_BYTES."""
    lib = H.lib()
    cap = H.noalloc_scratch_bytes()
    assert cap == 32 * 1024 * 1024
    p, r = _pages(), _recs()
    call = lambda sh=_shape(), crc=FAKE, table=FAKE, rr=r: lib.hkv_quant_fp8_crc_noalloc(
        ctypes.byref(sh), ctypes.byref(p), 0, ctypes.c_void_p(table), ctypes.byref(rr),
        ctypes.c_void_p(crc), None)
    assert call(crc=0) == H.ERR_INVALID_ARG
    assert call(table=0) == H.ERR_INVALID_ARG
    assert call(sh=_shape(head_dim=64)) == H.ERR_INVALID_ARG
    assert call(rr=_recs(base=FAKE + 8)) == H.ERR_INVALID_ARG
    # 80 layers x 1,024 blocks of 64 x 8 vectors: 341 MB of scratch needed
    big = _shape(n_layers=80, n_blocks=1024, block_tokens=64, n_kv_heads=8)
    rb = 133120
    assert lib.hkv_quant_crc_workspace_bytes(ctypes.byref(big), 0) > cap
    big_r = _recs(layer_stride_bytes=1024 * rb, block_stride_bytes=rb)
    assert call(sh=big, rr=big_r) == H.ERR_UNSUPPORTED
    # one such layer fits (4.3 MB); the largest fitting layer count is refused one above
    one = _shape(n_layers=1, n_blocks=1024, block_tokens=64, n_kv_heads=8)
    per_layer = lib.hkv_quant_crc_workspace_bytes(ctypes.byref(one), 0)
    assert per_layer == 1024 * (rb // 128) * 4 <= cap
    n_fit = cap // per_layer
    over = _shape(n_layers=n_fit + 1, n_blocks=1024, block_tokens=64, n_kv_heads=8)
    assert call(sh=over, rr=big_r) == H.ERR_UNSUPPORTED
    assert call(sh=_shape(n_blocks=0), crc=0, table=0) == H.OK    # empty: nothing launched


def test_staged_fetch_rejects_bad_arguments():
    """hkv_fetch_staged validates everything on the host before it creates an
    event or enqueues a copy."""
    lib = H.lib()
    s, p = _shape(), _pages()
    rb = 33280

    def call(sh=s, host=FAKE, ls=4 * rb, bs=rb, s0=FAKE + (1 << 24), s1=FAKE + (1 << 25),
             sb=4 * rb, table=FAKE, dm=FAKE, base=1e4, pairs=0, fmt=0, dt=0):
        hr = H.HostRecords(host, ls, bs)
        return lib.hkv_fetch_staged(ctypes.byref(sh), fmt, ctypes.byref(hr), ctypes.c_void_p(s0),
                                    ctypes.c_void_p(s1), sb, ctypes.c_void_p(table),
                                    ctypes.c_void_p(dm), None, base, pairs, ctypes.byref(p), dt,
                                    None, None, None)
    assert call(host=0) == H.ERR_INVALID_ARG
    assert call(host=FAKE + 8) == H.ERR_INVALID_ARG
    assert call(s0=0) == H.ERR_INVALID_ARG
    assert call(s1=FAKE + (1 << 24)) == H.ERR_INVALID_ARG          # the same buffer twice
    assert call(s1=FAKE + 8) == H.ERR_INVALID_ARG
    assert call(sb=4 * rb - 16) == H.ERR_INVALID_ARG               # smaller than one layer
    assert call(bs=rb - 16) == H.ERR_INVALID_ARG
    assert call(ls=3 * rb) == H.ERR_INVALID_ARG                     # layers overlap
    assert call(ls=-16) == H.ERR_INVALID_ARG
    assert call(fmt=5) == H.ERR_INVALID_ARG
    assert call(base=0.0) == H.ERR_INVALID_ARG
    assert call(pairs=3) == H.ERR_INVALID_ARG
    assert call(table=0) == H.ERR_INVALID_ARG
    assert call(dm=0) == H.ERR_INVALID_ARG
    assert call(dt=7) == H.ERR_INVALID_ARG
    assert call(sh=_shape(head_dim=64)) == H.ERR_INVALID_ARG
    assert call(sh=_shape(n_layers=0)) == H.OK                      # empty: nothing enqueued
    assert call(sh=_shape(n_blocks=0), table=0, dm=0) == H.OK


def test_staged_binding_checks_host_memory():
    import torch
    k = torch.zeros((1, 4, 16, 8, 128), dtype=torch.bfloat16)
    host = torch.zeros((1, 4, 33280), dtype=torch.uint8)           # not pinned (no GPU here)
    with pytest.raises(ValueError, match="pinned"):
        H.fetch_staged(host, "fp8", torch.zeros(4, dtype=torch.int32),
                       torch.zeros(4, dtype=torch.int32), 1e4, "interleaved", k, k,
                       (torch.zeros(1, dtype=torch.uint8),) * 2)


def test_binding_checks_record_size():
    """A records tensor whose last axis is shorter than one record of the
    call's format and shape is refused by the binding (the library can only
    compare strides, and a single record has none)."""
    import torch
    int4_rec = torch.zeros((1, 1, H.record_bytes("int4", 16, 8)), dtype=torch.uint8)
    fp8_rec = torch.zeros((1, 1, H.record_bytes("fp8", 16, 8)), dtype=torch.uint8)
    with pytest.raises(ValueError, match="needs 33280"):
        H._records(int4_rec, "fp8", 16, 8)
    assert H._records(fp8_rec, "fp8", 16, 8).base == fp8_rec.data_ptr()
    assert H._records(fp8_rec, "int4", 16, 8).block_stride_bytes == fp8_rec.stride(1)
    with pytest.raises(ValueError, match="needs 33344"):          # a frame: 64 + record
        H._records(fp8_rec, "fp8", 16, 8, header=64)


def test_stream_probe_rejects_bad_arguments():
    lib = H.lib()
    call = lambda src=FAKE, dst=FAKE + (1 << 20), n=1024: lib.hkv_stream_probe(
        ctypes.c_void_p(src), ctypes.c_void_p(dst), n, None)
    assert call(n=1000) == H.ERR_INVALID_ARG          # not a multiple of 128
    assert call(n=-128) == H.ERR_INVALID_ARG
    assert call(src=0) == H.ERR_INVALID_ARG
    assert call(dst=FAKE + 8) == H.ERR_INVALID_ARG
    assert call(n=0, src=0, dst=0) == H.OK


def test_stream_probe_put_rejects_bad_arguments():
    lib = H.lib()
    call = lambda src=FAKE, dst=FAKE + (1 << 20), n=1024: lib.hkv_stream_probe_put(
        ctypes.c_void_p(src), ctypes.c_void_p(dst), n, None)
    assert call(n=1000) == H.ERR_INVALID_ARG          # not a multiple of 128
    assert call(n=-128) == H.ERR_INVALID_ARG
    assert call(src=0) == H.ERR_INVALID_ARG
    assert call(src=FAKE + 8) == H.ERR_INVALID_ARG
    assert call(dst=FAKE + 8) == H.ERR_INVALID_ARG
    assert call(n=128 * ((1 << 28) + 1)) == H.ERR_UNSUPPORTED   # more rows than the grid holds
    assert call(n=0, src=0, dst=0) == H.OK


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: with the shared library absent every call raises instead
    of computing anything another way."""
    monkeypatch.setattr(hkv, "LIB_PATH", str(tmp_path / "libhkv_absent.so"))
    monkeypatch.setattr(hkv, "_lib", None)
    with pytest.raises(ImportError, match="not built"):
        hkv.lib()
    with pytest.raises(ImportError):
        hkv.record_bytes("fp8", 64, 8)


def test_binding_requires_gpu_tensors():
    """Host tensors never reach the library: their addresses would be
    dereferenced by kernels."""
    import torch
    k = torch.zeros((1, 4, 16, 8, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="on a GPU"):
        H.quant_fp8(k, k, torch.arange(4, dtype=torch.int32),
                    torch.zeros((1, 4, 33280), dtype=torch.uint8))
    with pytest.raises(ValueError, match="on a GPU"):
        H.token_drift(torch.zeros((4, 64)), torch.zeros((4, 64)))
    with pytest.raises(ValueError, match="on a GPU"):
        H.select_top_tokens(torch.zeros(64), 8)


def test_views_beyond_the_address_space_are_rejected():
    """A view whose largest addressed byte offset reaches 2^47 (more than a
    device can address, so no valid buffer) is refused before any launch:
    the kernels' 64-bit offset arithmetic can then never overflow."""
    lib = H.lib()
    big = 1 << 47
    s = _shape()                                   # 2 layers, 4 blocks of 16 x 8, fp32 pages
    # pages: one layer stride of 2^47 bytes (fp32: 2^45 elements)
    assert _quant(s, _pages(layer_stride=big // 4), 0, FAKE, _recs()) == H.ERR_INVALID_ARG
    # the same just below the limit passes the checks (an empty call then launches nothing)
    assert _quant(_shape(n_blocks=0), _pages(layer_stride=(big - (1 << 20)) // 4), 0, 0,
                  _recs()) == H.OK
    # pages: the page stride over num_pages, the token and head strides
    assert _quant(s, _pages(page_stride=big // 8), 0, FAKE, _recs()) == H.ERR_INVALID_ARG
    assert _quant(_shape(block_tokens=2), _pages(token_stride=big // 4), 0, FAKE,
                  _recs(layer_stride_bytes=4 * 4160, block_stride_bytes=4160)) == \
        H.ERR_INVALID_ARG
    assert _quant(_shape(n_kv_heads=2, block_tokens=8), _pages(head_stride=big // 4), 0, FAKE,
                  _recs(layer_stride_bytes=4 * 4160, block_stride_bytes=4160)) == \
        H.ERR_INVALID_ARG
    # records: block and layer strides
    assert _quant(s, _pages(), 0, FAKE, _recs(block_stride_bytes=big // 2)) == H.ERR_INVALID_ARG
    assert _quant(s, _pages(), 0, FAKE, _recs(layer_stride_bytes=big)) == H.ERR_INVALID_ARG
    # fetch: the destination pages and the records
    assert _fetch(s, _recs(), FAKE, FAKE, 1e4, 0, _pages(layer_stride=big // 4), 0) == \
        H.ERR_INVALID_ARG
    assert _fetch(s, _recs(block_stride_bytes=big // 2), FAKE, FAKE, 1e4, 0, _pages(), 0) == \
        H.ERR_INVALID_ARG
    # CRC over records
    assert lib.hkv_crc32_blocks(ctypes.byref(s), 0, ctypes.byref(_recs(layer_stride_bytes=big)),
                                ctypes.c_void_p(FAKE), None) == H.ERR_INVALID_ARG
    # frames
    assert lib.hkv_frame_verify(ctypes.byref(s), 0,
                                ctypes.byref(_frames_view(block_stride_bytes=big // 2)), 0,
                                ctypes.c_void_p(FAKE), None) == H.ERR_INVALID_ARG
    # drift rows (bf16: 2^46 elements per row is 2^47 bytes)
    assert _drift(stride=big // 2) == H.ERR_INVALID_ARG
    # staged fetch: the host records and every layer's destination pages
    rb = 33280

    def staged(ls=4 * rb, pages=_pages()):
        hr = H.HostRecords(FAKE, ls, rb)
        return lib.hkv_fetch_staged(ctypes.byref(s), 0, ctypes.byref(hr),
                                    ctypes.c_void_p(FAKE + (1 << 24)),
                                    ctypes.c_void_p(FAKE + (1 << 25)), 4 * rb,
                                    ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None, 1e4, 0,
                                    ctypes.byref(pages), 0, None, None, None)
    assert staged(ls=big) == H.ERR_INVALID_ARG
    assert staged(pages=_pages(layer_stride=big // 4)) == H.ERR_INVALID_ARG
