"""Thin ctypes binding of libhkv (include/hkv.h).

Argument marshalling only: every step of put, CRC and fetch runs in the HIP
kernels of libhkv.so.  torch is used for device memory and streams: tensors
supply device pointers and strides, and calls are enqueued on the caller's
current torch stream unless another is given.

There is no fallback: if libhkv.so is missing or cannot be loaded, importing
the library raises.
"""

from __future__ import annotations

import ctypes
import functools
import os
import re

import torch  # load torch's HIP runtime first so libhkv binds to the same one

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhkv.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "hkv.h")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP = 0, -1, -2, -3
F32, F16, BF16 = 0, 1, 2
FP8_E4M3, INT4 = 0, 1
ROPE_INTERLEAVED, ROPE_HALF_SPLIT = 0, 1
HEAD_DIM = 128

FORMATS = {"fp8": FP8_E4M3, "int4": INT4, FP8_E4M3: FP8_E4M3, INT4: INT4}
PAIRS = {"interleaved": ROPE_INTERLEAVED, "half_split": ROPE_HALF_SPLIT,
         ROPE_INTERLEAVED: ROPE_INTERLEAVED, ROPE_HALF_SPLIT: ROPE_HALF_SPLIT}
TORCH_DTYPES = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}


class HkvError(RuntimeError):
    def __init__(self, call, status):
        self.status = status
        super().__init__(f"{call} failed: {status_string(status)} ({status})")


class Shape(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_blocks", ctypes.c_int32),
                ("block_tokens", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32)]


class Pages(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("layer_stride", ctypes.c_int64), ("page_stride", ctypes.c_int64),
                ("token_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
                ("num_pages", ctypes.c_int32)]


class Records(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("layer_stride_bytes", ctypes.c_int64),
                ("block_stride_bytes", ctypes.c_int64)]


class HostRecords(ctypes.Structure):
    _fields_ = [("host_base", ctypes.c_void_p), ("layer_stride_bytes", ctypes.c_int64),
                ("block_stride_bytes", ctypes.c_int64)]


_lib = None


def declared_symbols():
    """Names of the functions include/hkv.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hkv_[a-z0-9_]+)\s*\(", text)))


def _header_define(name: str) -> int:
    """An integer #define of include/hkv.h (e.g. HKV_NOALLOC_SCRATCH_BYTES)."""
    with open(HEADER) as f:
        m = re.search(r"#define\s+" + name + r"\s+\(?([0-9LL*\s]+)\)?", f.read())
    if m is None:
        raise KeyError(name)
    value = 1
    for factor in m.group(1).replace("LL", "").split("*"):
        value *= int(factor)
    return value


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run "
                              "`python -m quantization_rope_reuse_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp = ctypes.c_void_p
        l.hkv_quant_fp8.argtypes = [P(Shape), P(Pages), ctypes.c_int32, vp, P(Records), vp]
        l.hkv_quant_int4.argtypes = [P(Shape), P(Pages), ctypes.c_int32, vp, P(Records), vp]
        l.hkv_quant_fp8_crc.argtypes = [P(Shape), P(Pages), ctypes.c_int32, vp, P(Records), vp,
                                        vp, ctypes.c_int64, vp, vp]
        l.hkv_quant_int4_crc.argtypes = l.hkv_quant_fp8_crc.argtypes
        l.hkv_quant_fp8_crc_noalloc.argtypes = [P(Shape), P(Pages), ctypes.c_int32, vp,
                                                P(Records), vp, vp]
        l.hkv_quant_crc_workspace_bytes.argtypes = [P(Shape), ctypes.c_int32]
        l.hkv_quant_crc_workspace_bytes.restype = ctypes.c_int64
        l.hkv_fetch_dequant_rope_shift.argtypes = [
            P(Shape), ctypes.c_int32, P(Records), vp, vp, vp, ctypes.c_double, ctypes.c_int32,
            P(Pages), ctypes.c_int32, vp]
        l.hkv_fetch_dequant_rope_shift_tokens.argtypes = [
            P(Shape), ctypes.c_int32, P(Records), vp, vp, vp, ctypes.c_double, ctypes.c_int32,
            P(Pages), ctypes.c_int32, vp]
        l.hkv_fetch_staged.argtypes = [
            P(Shape), ctypes.c_int32, P(HostRecords), vp, vp, ctypes.c_int64, vp, vp, vp,
            ctypes.c_double, ctypes.c_int32, P(Pages), ctypes.c_int32, vp, vp, vp]
        l.hkv_page_visit_order.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, vp, vp]
        l.hkv_crc32_blocks.argtypes = [P(Shape), ctypes.c_int32, P(Records), vp, vp]
        l.hkv_token_drift.argtypes = [vp, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                      ctypes.c_int32, vp, vp]
        l.hkv_select_top_tokens.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, vp, vp,
                                            ctypes.c_int64, vp]
        l.hkv_select_workspace_bytes.argtypes = [ctypes.c_int32]
        l.hkv_select_workspace_bytes.restype = ctypes.c_int64
        l.hkv_frame_headers.argtypes = [P(Shape), ctypes.c_int32, P(Records), vp, vp,
                                        ctypes.c_int32, vp]
        l.hkv_frame_verify.argtypes = [P(Shape), ctypes.c_int32, P(Records), ctypes.c_int32,
                                       vp, vp]
        l.hkv_frame_delta_m.argtypes = [P(Shape), ctypes.c_int32, P(Records), vp, vp, vp]
        l.hkv_stream_probe.argtypes = [vp, vp, ctypes.c_int64, vp]
        l.hkv_stream_probe.restype = ctypes.c_int
        l.hkv_stream_probe_put.argtypes = [vp, vp, ctypes.c_int64, vp]
        l.hkv_stream_probe_put.restype = ctypes.c_int
        l.hkv_stream_pair_create.argtypes = [ctypes.c_int32, P(vp), P(vp)]
        l.hkv_stream_pair_create.restype = ctypes.c_int
        l.hkv_stream_destroy.argtypes = [vp]
        l.hkv_stream_destroy.restype = ctypes.c_int
        for name in ("hkv_quant_fp8", "hkv_quant_int4", "hkv_quant_fp8_crc",
                     "hkv_quant_int4_crc", "hkv_quant_fp8_crc_noalloc",
                     "hkv_fetch_dequant_rope_shift",
                     "hkv_fetch_dequant_rope_shift_tokens", "hkv_fetch_staged",
                     "hkv_crc32_blocks",
                     "hkv_page_visit_order", "hkv_token_drift", "hkv_select_top_tokens",
                     "hkv_frame_headers", "hkv_frame_verify", "hkv_frame_delta_m"):
            getattr(l, name).restype = ctypes.c_int
        l.hkv_record_bytes.argtypes = [ctypes.c_int32] * 4
        l.hkv_record_bytes.restype = ctypes.c_int64
        l.hkv_status_string.argtypes = [ctypes.c_int32]
        l.hkv_status_string.restype = ctypes.c_char_p
        _lib = l
    return _lib


def status_string(status: int) -> str:
    return lib().hkv_status_string(int(status)).decode()


def record_bytes(fmt, block_tokens: int, n_kv_heads: int, head_dim: int = HEAD_DIM) -> int:
    return int(lib().hkv_record_bytes(FORMATS[fmt], block_tokens, n_kv_heads, head_dim))


# ---------------------------------------------------------------------------
# Marshalling helpers
# ---------------------------------------------------------------------------

def _stream(stream, device):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _as5d(t: torch.Tensor) -> torch.Tensor:
    """Pages as [L, P, T_b, H, 128]; a 4-D tensor is one layer."""
    if t.dim() == 4:
        return t.unsqueeze(0)
    if t.dim() != 5:
        raise ValueError("pages must be [L, P, T_b, H, 128] or [P, T_b, H, 128]")
    return t


def _pages(k: torch.Tensor, v: torch.Tensor):
    k5, v5 = _as5d(k), _as5d(v)
    if k5.shape != v5.shape or k5.stride() != v5.stride() or k5.dtype != v5.dtype:
        raise ValueError("K and V pages must share shape, strides and dtype")
    if k5.shape[-1] != HEAD_DIM or k5.stride(-1) != 1:
        raise ValueError("the last (head_dim=128) axis of the pages must be contiguous")
    if k5.dtype not in TORCH_DTYPES:
        raise ValueError(f"unsupported page dtype {k5.dtype}")
    s = k5.stride()
    p = Pages(k5.data_ptr(), v5.data_ptr(), s[0], s[1], s[2], s[3], k5.shape[1])
    return p, k5.shape, TORCH_DTYPES[k5.dtype]


def _records(r: torch.Tensor, fmt, block_tokens: int, n_kv_heads: int, header: int = 0):
    """Records as a uint8 tensor [L, n_blocks, >= header + record_bytes]: the
    last axis must hold a whole record of this format and shape (and the
    header, for frames), since the library can only compare strides."""
    if r.dtype != torch.uint8 or r.dim() != 3 or r.stride(2) != 1:
        raise ValueError("records must be a uint8 [L, n_blocks, bytes] tensor, last axis contiguous")
    need = header + record_bytes(fmt, block_tokens, n_kv_heads)
    if r.shape[2] < need:
        raise ValueError(f"records hold {r.shape[2]} bytes per block; a {fmt} record of "
                         f"{block_tokens} tokens x {n_kv_heads} heads needs {need}")
    return Records(r.data_ptr(), r.stride(0), r.stride(1))


def _i32(t: torch.Tensor, name: str):
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor")
    return ctypes.c_void_p(t.data_ptr())


def _check(call: str, status: int):
    if status != OK:
        raise HkvError(call, status)


def _on_one_gpu(fn):
    """Every tensor argument of a call must be a GPU tensor and all of them on
    one device: the kernels dereference their addresses."""
    @functools.wraps(fn)
    def checked(*args, **kwargs):
        dev = None
        for a in (*args, *kwargs.values()):
            if isinstance(a, torch.Tensor):
                if a.device.type != "cuda":
                    raise ValueError(f"{fn.__name__}: tensor arguments must be on a GPU, "
                                     f"got one on {a.device}")
                if dev is None:
                    dev = a.device
                elif a.device != dev:
                    raise ValueError(f"{fn.__name__}: tensor arguments on {dev} and {a.device}")
        return fn(*args, **kwargs)
    return checked


def alloc_records(n_layers: int, n_blocks: int, fmt, block_tokens: int, n_kv_heads: int,
                  device="cuda"):
    """A uint8 [L, n_blocks, record_bytes] tensor (block stride rounded up to 16)."""
    rb = record_bytes(fmt, block_tokens, n_kv_heads)
    stride = (rb + 15) // 16 * 16
    buf = torch.empty((n_layers, n_blocks, stride), dtype=torch.uint8, device=device)
    return buf[:, :, :rb]


# ---------------------------------------------------------------------------
# The four calls
# ---------------------------------------------------------------------------

def _quant(name, fmt, k_pages, v_pages, block_table, records, stream):
    pages, shp, dt = _pages(k_pages, v_pages)
    L, _, tb, H, d = shp
    if records.shape[0] != L or records.shape[1] != block_table.numel():
        raise ValueError("records must be [L, n_blocks, bytes] matching pages and table")
    shape = Shape(L, block_table.numel(), tb, H, d)
    rec = _records(records, fmt, tb, H)
    st = getattr(lib(), name)(ctypes.byref(shape), ctypes.byref(pages), dt,
                              _i32(block_table, "block_table"), ctypes.byref(rec),
                              _stream(stream, k_pages.device))
    _check(name, st)
    return records


@_on_one_gpu
def quant_fp8(k_pages, v_pages, block_table, records, stream=None):
    """Quantize the blocks k/v_pages[:, block_table[b]] into records[:, b] (FP8)."""
    return _quant("hkv_quant_fp8", "fp8", k_pages, v_pages, block_table, records, stream)


@_on_one_gpu
def quant_int4(k_pages, v_pages, block_table, records, stream=None):
    """Quantize the blocks k/v_pages[:, block_table[b]] into records[:, b] (INT4)."""
    return _quant("hkv_quant_int4", "int4", k_pages, v_pages, block_table, records, stream)


def quant_crc_workspace_bytes(fmt, n_layers: int, n_blocks: int, block_tokens: int,
                              n_kv_heads: int) -> int:
    shape = Shape(n_layers, n_blocks, block_tokens, n_kv_heads, HEAD_DIM)
    return int(lib().hkv_quant_crc_workspace_bytes(ctypes.byref(shape), FORMATS[fmt]))


@_on_one_gpu
def quant_crc(fmt, k_pages, v_pages, block_table, records, crc_out=None, workspace=True,
              stream=None, records_ready=None):
    """Put (FP8 or INT4) and the CRC-32 of every written record in one pass.
    Returns crc_out, an int32 tensor [L, n_blocks] holding uint32 values.
    workspace: True (allocated here), or a uint8 tensor of at least
    quant_crc_workspace_bytes bytes.  records_ready: None, or a
    torch.cuda.Event that the library records on the stream once the
    records are written, before the CRC merge (other streams that need only
    the records wait on it)."""
    pages, shp, dt = _pages(k_pages, v_pages)
    L, _, tb, H, d = shp
    nb = block_table.numel()
    if records.shape[0] != L or records.shape[1] != nb:
        raise ValueError("records must be [L, n_blocks, bytes] matching pages and table")
    if crc_out is None:
        crc_out = torch.empty((L, nb), dtype=torch.int32, device=records.device)
    if crc_out.dtype != torch.int32 or not crc_out.is_contiguous() or crc_out.numel() != L * nb:
        raise ValueError("crc_out must be a contiguous int32 tensor of L * n_blocks elements")
    need = quant_crc_workspace_bytes(fmt, L, nb, tb, H)
    if workspace is True:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=records.device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    shape = Shape(L, nb, tb, H, d)
    rec = _records(records, fmt, tb, H)
    hs = _stream(stream, k_pages.device)
    ready = None
    if records_ready is not None:
        if not records_ready.cuda_event:     # torch creates its events on first record
            records_ready.record(torch.cuda.current_stream(k_pages.device))
        ready = ctypes.c_void_p(records_ready.cuda_event)
    name = "hkv_quant_fp8_crc" if FORMATS[fmt] == FP8_E4M3 else "hkv_quant_int4_crc"
    st = getattr(lib(), name)(ctypes.byref(shape), ctypes.byref(pages), dt,
                              _i32(block_table, "block_table"), ctypes.byref(rec),
                              ctypes.c_void_p(crc_out.data_ptr()),
                              ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), hs, ready)
    _check(name, st)
    return crc_out


NOALLOC_SCRATCH_BYTES = None     # HKV_NOALLOC_SCRATCH_BYTES, read from the header


@_on_one_gpu
def quant_fp8_crc_noalloc(k_pages, v_pages, block_table, records, crc_out, stream=None):
    """hkv_quant_fp8_crc_noalloc: the FP8 put and the CRC-32 of every written
    record in one pass, in the library's per-GPU scratch array (nothing is
    allocated, here or in the library).  crc_out: a contiguous int32 tensor
    of L * n_blocks elements (uint32 values), which the caller provides.
    Shapes that need more than HKV_NOALLOC_SCRATCH_BYTES of scratch raise
    HkvError (HKV_ERR_UNSUPPORTED) before anything runs.  Calls that overlap
    in time on one GPU share its scratch and must not be made."""
    pages, shp, dt = _pages(k_pages, v_pages)
    L, _, tb, H, d = shp
    nb = block_table.numel()
    if records.shape[0] != L or records.shape[1] != nb:
        raise ValueError("records must be [L, n_blocks, bytes] matching pages and table")
    if crc_out.dtype != torch.int32 or not crc_out.is_contiguous() or crc_out.numel() != L * nb:
        raise ValueError("crc_out must be a contiguous int32 tensor of L * n_blocks elements")
    shape = Shape(L, nb, tb, H, d)
    rec = _records(records, "fp8", tb, H)
    st = lib().hkv_quant_fp8_crc_noalloc(ctypes.byref(shape), ctypes.byref(pages), dt,
                                         _i32(block_table, "block_table"), ctypes.byref(rec),
                                         ctypes.c_void_p(crc_out.data_ptr()),
                                         _stream(stream, k_pages.device))
    _check("hkv_quant_fp8_crc_noalloc", st)
    return crc_out


def noalloc_scratch_bytes() -> int:
    """HKV_NOALLOC_SCRATCH_BYTES of include/hkv.h."""
    global NOALLOC_SCRATCH_BYTES
    if NOALLOC_SCRATCH_BYTES is None:
        NOALLOC_SCRATCH_BYTES = _header_define("HKV_NOALLOC_SCRATCH_BYTES")
    return NOALLOC_SCRATCH_BYTES


def _fetch(name, records, fmt, block_table, delta, n_delta, rope_base, pairs, k_pages, v_pages,
           visit_order, stream):
    pages, shp, dt = _pages(k_pages, v_pages)
    L, _, tb, H, d = shp
    nb = block_table.numel()
    if records.shape[0] != L or records.shape[1] != nb or delta.numel() != n_delta(nb, tb):
        raise ValueError("records [L, n_blocks, bytes], table and deltas must agree")
    if visit_order is not None and visit_order.numel() != nb:
        raise ValueError("visit_order must hold n_blocks entries")
    shape = Shape(L, nb, tb, H, d)
    rec = _records(records, fmt, tb, H)
    order = None if visit_order is None else _i32(visit_order, "visit_order")
    st = getattr(lib(), name)(
        ctypes.byref(shape), FORMATS[fmt], ctypes.byref(rec), _i32(block_table, "block_table"),
        _i32(delta, "delta_m"), order, float(rope_base), PAIRS[pairs], ctypes.byref(pages),
        dt, _stream(stream, k_pages.device))
    _check(name, st)
    return k_pages, v_pages


@_on_one_gpu
def fetch_dequant_rope_shift(records, fmt, block_table, delta_m, rope_base, pairs,
                             k_pages, v_pages, visit_order=None, stream=None):
    """Dequantize records[:, b], shift keys by delta_m[b], store at page
    block_table[b] of k/v_pages (dtype of the pages).  visit_order: optional
    int32 permutation of the blocks (see page_visit_order)."""
    return _fetch("hkv_fetch_dequant_rope_shift", records, fmt, block_table, delta_m,
                  lambda nb, tb: nb, rope_base, pairs, k_pages, v_pages, visit_order, stream)


@_on_one_gpu
def fetch_dequant_rope_shift_tokens(records, fmt, block_table, delta_m_tokens, rope_base, pairs,
                                    k_pages, v_pages, visit_order=None, stream=None):
    """As fetch_dequant_rope_shift with one delta per token: delta_m_tokens
    is an int32 [n_blocks, block_tokens] tensor."""
    return _fetch("hkv_fetch_dequant_rope_shift_tokens", records, fmt, block_table,
                  delta_m_tokens, lambda nb, tb: nb * tb, rope_base, pairs, k_pages, v_pages,
                  visit_order, stream)


def fetch_staged(host_records, fmt, block_table, delta_m, rope_base, pairs, k_pages, v_pages,
                 staging, visit_order=None, copy_stream=None, fetch_stream=None,
                 layer_ready=None):
    """Layer-by-layer fetch from host memory through two staging buffers
    (hkv_fetch_staged): layer l's records are copied from host_records (a
    pinned CPU uint8 tensor [L, n_blocks, >= record_bytes]) into staging[l %
    2] on copy_stream, then fetched into layer l of k/v_pages on
    fetch_stream.  staging: two device uint8 tensors, each holding one
    layer's records.  layer_ready: None or L torch.cuda.Event objects,
    recorded on fetch_stream after each layer's fetch.  Streams default to
    the current one (copies and fetches then do not overlap)."""
    if not isinstance(host_records, torch.Tensor) or host_records.device.type != "cpu":
        raise ValueError("host_records must be a CPU tensor")
    if not host_records.is_pinned():
        raise ValueError("host_records must be in pinned host memory (pin_memory())")
    if host_records.dim() != 3 or host_records.stride(2) != 1 or host_records.dtype != torch.uint8:
        raise ValueError("host_records must be a uint8 [L, n_blocks, bytes] tensor, last axis "
                         "contiguous")
    if len(staging) != 2:
        raise ValueError("staging must be two device buffers")
    dev = k_pages.device
    for t in (block_table, delta_m, k_pages, v_pages, *staging,
              *(() if visit_order is None else (visit_order,))):
        if not isinstance(t, torch.Tensor) or t.device != dev or dev.type != "cuda":
            raise ValueError("staging, tables and pages must be tensors on one GPU")
    pages, shp, dt = _pages(k_pages, v_pages)
    L, _, tb, H, d = shp
    nb = block_table.numel()
    if host_records.shape[0] != L or host_records.shape[1] != nb or delta_m.numel() != nb:
        raise ValueError("host records [L, n_blocks, bytes], pages, table and deltas must agree")
    need = record_bytes(fmt, tb, H)
    if host_records.shape[2] < need:
        raise ValueError(f"host records hold {host_records.shape[2]} bytes per block; "
                         f"needs {need}")
    extent = (nb - 1) * host_records.stride(1) + need
    for b in staging:
        if b.dtype != torch.uint8 or not b.is_contiguous() or b.numel() < extent:
            raise ValueError(f"each staging buffer must be a contiguous uint8 tensor of at "
                             f"least {extent} bytes")
    if visit_order is not None and visit_order.numel() != nb:
        raise ValueError("visit_order must hold n_blocks entries")
    fetch_stream = fetch_stream or torch.cuda.current_stream(dev)
    copy_stream = copy_stream or fetch_stream
    events = None
    if layer_ready is not None:
        if len(layer_ready) != L:
            raise ValueError("layer_ready must hold one event per layer")
        for ev in layer_ready:
            if not ev.cuda_event:            # torch creates its events on first record
                ev.record(fetch_stream)
        events = (ctypes.c_void_p * L)(*[ev.cuda_event for ev in layer_ready])
    shape = Shape(L, nb, tb, H, d)
    hr = HostRecords(host_records.data_ptr(), host_records.stride(0), host_records.stride(1))
    order = None if visit_order is None else _i32(visit_order, "visit_order")
    st = lib().hkv_fetch_staged(
        ctypes.byref(shape), FORMATS[fmt], ctypes.byref(hr),
        ctypes.c_void_p(staging[0].data_ptr()), ctypes.c_void_p(staging[1].data_ptr()),
        min(staging[0].numel(), staging[1].numel()), _i32(block_table, "block_table"),
        _i32(delta_m, "delta_m"), order, float(rope_base), PAIRS[pairs], ctypes.byref(pages),
        dt, _stream(copy_stream, dev), _stream(fetch_stream, dev),
        None if events is None else ctypes.cast(events, ctypes.c_void_p))
    _check("hkv_fetch_staged", st)
    return k_pages, v_pages


def alloc_staging(n_blocks: int, fmt, block_tokens: int, n_kv_heads: int, device="cuda"):
    """Two device buffers, each holding one layer of records laid out as
    alloc_records lays them out (block stride rounded up to 16 bytes)."""
    stride = (record_bytes(fmt, block_tokens, n_kv_heads) + 15) // 16 * 16
    return tuple(torch.empty(n_blocks * stride, dtype=torch.uint8, device=device)
                 for _ in range(2))


@_on_one_gpu
def page_visit_order(block_table, num_pages: int, out=None, stream=None):
    """Blocks listed by increasing destination page (skipped blocks last):
    an int32 tensor [n_blocks] for fetch_dequant_rope_shift's visit_order."""
    nb = block_table.numel()
    if out is None:
        out = torch.empty(nb, dtype=torch.int32, device=block_table.device)
    if out.numel() != nb:
        raise ValueError("out must hold n_blocks entries")
    st = lib().hkv_page_visit_order(_i32(block_table, "block_table"), nb, int(num_pages),
                                    _i32(out, "out"), _stream(stream, block_table.device))
    _check("hkv_page_visit_order", st)
    return out


class StreamPair:
    """Two CU-partitioned streams (hkv_stream_pair_create) as torch streams:
    `fetch` with fetch_cus compute units, `compute` with the rest."""

    def __init__(self, fetch_cus: int, device=None):
        f, c = ctypes.c_void_p(), ctypes.c_void_p()
        _check("hkv_stream_pair_create",
               lib().hkv_stream_pair_create(int(fetch_cus), ctypes.byref(f), ctypes.byref(c)))
        self._handles = (f.value, c.value)
        self.fetch = torch.cuda.ExternalStream(f.value, device=device)
        self.compute = torch.cuda.ExternalStream(c.value, device=device)

    def close(self):
        if self._handles:
            torch.cuda.synchronize()
            for h in self._handles:
                lib().hkv_stream_destroy(ctypes.c_void_p(h))
            self._handles = None


@_on_one_gpu
def crc32_blocks(records, fmt, block_tokens: int, n_kv_heads: int, out=None, stream=None):
    """CRC-32 of every record; returns a uint32-valued int32 tensor [L, n_blocks]
    (use `.view(torch.uint32)` or mask with 0xFFFFFFFF after widening)."""
    L, nb = records.shape[0], records.shape[1]
    if out is None:
        out = torch.empty((L, nb), dtype=torch.int32, device=records.device)
    if out.dtype != torch.int32 or not out.is_contiguous() or out.numel() != L * nb:
        raise ValueError("out must be a contiguous int32 tensor of L * n_blocks elements")
    shape = Shape(L, nb, block_tokens, n_kv_heads, HEAD_DIM)
    rec = _records(records, fmt, block_tokens, n_kv_heads)
    st = lib().hkv_crc32_blocks(ctypes.byref(shape), FORMATS[fmt], ctypes.byref(rec),
                                ctypes.c_void_p(out.data_ptr()), _stream(stream, records.device))
    _check("hkv_crc32_blocks", st)
    return out


@_on_one_gpu
def token_drift(h_cached, h_fresh, out=None, stream=None):
    """Per-token drift ||h_fresh[t] - h_cached[t]||_2 of two [n_tokens, d_model]
    tensors (same dtype, same row stride, last axis contiguous); returns a
    float32 tensor [n_tokens]."""
    if h_cached.shape != h_fresh.shape or h_cached.dim() != 2:
        raise ValueError("hidden states must be two [n_tokens, d_model] tensors of one shape")
    if h_cached.dtype != h_fresh.dtype or h_cached.dtype not in TORCH_DTYPES:
        raise ValueError("hidden states must share an f32/f16/bf16 dtype")
    if h_cached.stride() != h_fresh.stride() or (h_cached.shape[1] > 1 and h_cached.stride(1) != 1):
        raise ValueError("hidden states must share row strides, last axis contiguous")
    n, d = h_cached.shape
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=h_cached.device)
    if out.dtype != torch.float32 or not out.is_contiguous() or out.numel() != n:
        raise ValueError("out must be a contiguous float32 tensor of n_tokens elements")
    st = lib().hkv_token_drift(ctypes.c_void_p(h_cached.data_ptr()),
                               ctypes.c_void_p(h_fresh.data_ptr()), n, d,
                               h_cached.stride(0), TORCH_DTYPES[h_cached.dtype],
                               ctypes.c_void_p(out.data_ptr()), _stream(stream, h_cached.device))
    _check("hkv_token_drift", st)
    return out


def select_workspace_bytes(n_tokens: int) -> int:
    return int(lib().hkv_select_workspace_bytes(int(n_tokens)))


@_on_one_gpu
def select_top_tokens(drift, k: int, out=None, workspace=True, stream=None):
    """Indices of the k largest drift values, increasing; int32 tensor [k].
    workspace: True (a device buffer of select_workspace_bytes is allocated
    here: the many-workgroup path), None/False (one workgroup), or a uint8
    tensor to use as the workspace."""
    if drift.dtype != torch.float32 or not drift.is_contiguous():
        raise ValueError("drift must be a contiguous float32 tensor")
    n = drift.numel()
    if out is None:
        out = torch.empty(max(int(k), 0), dtype=torch.int32, device=drift.device)
    if out.numel() < k:
        raise ValueError("out must hold k entries")
    if workspace is True:
        workspace = torch.empty(max(select_workspace_bytes(n), 16), dtype=torch.uint8,
                                device=drift.device)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None and workspace is not False:
        if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor")
        ws_ptr, ws_bytes = ctypes.c_void_p(workspace.data_ptr()), workspace.numel()
    st = lib().hkv_select_top_tokens(ctypes.c_void_p(drift.data_ptr()), n, int(k),
                                     _i32(out, "out"), ws_ptr, ws_bytes,
                                     _stream(stream, drift.device))
    _check("hkv_select_top_tokens", st)
    return out


FRAME_HEADER_BYTES = 64
FRAME_BAD_MAGIC, FRAME_BAD_HEADER_CRC, FRAME_BAD_GEOMETRY = 1, 2, 4
FRAME_BAD_INDEX, FRAME_BAD_PAYLOAD_CRC = 8, 16


def alloc_frames(n_layers: int, n_blocks: int, fmt, block_tokens: int, n_kv_heads: int,
                 device="cuda"):
    """A uint8 [L, n_blocks, 64 + record_bytes] tensor of frames.  The frame
    stride is a multiple of 128 bytes and the frames start 64 bytes into a
    128-byte aligned allocation, so every record starts on a 128-byte line."""
    fb = FRAME_HEADER_BYTES + record_bytes(fmt, block_tokens, n_kv_heads)
    stride = (fb + 127) // 128 * 128
    n = n_layers * n_blocks * stride
    buf = torch.empty(n + 128, dtype=torch.uint8, device=device)
    skip = (64 - buf.data_ptr()) % 128
    return buf[skip:skip + n].view(n_layers, n_blocks, stride)[:, :, :fb]


def frame_records(frames):
    """The records inside frames: a view for the put, CRC and fetch calls."""
    return frames[:, :, FRAME_HEADER_BYTES:]


def _frame_args(frames, fmt, block_tokens, n_kv_heads):
    if frames.dim() != 3:
        raise ValueError("frames must be a uint8 [L, n_blocks, bytes] tensor")
    shape = Shape(frames.shape[0], frames.shape[1], block_tokens, n_kv_heads, HEAD_DIM)
    return shape, _records(frames, fmt, block_tokens, n_kv_heads, header=FRAME_HEADER_BYTES)


@_on_one_gpu
def frame_headers(frames, fmt, block_tokens: int, n_kv_heads: int, crc, m_old,
                  layer_base: int = 0, stream=None):
    """Write the header of every frame (records and their CRCs already there)."""
    shape, fr = _frame_args(frames, fmt, block_tokens, n_kv_heads)
    if crc.numel() != frames.shape[0] * frames.shape[1] or m_old.numel() != frames.shape[1]:
        raise ValueError("crc must hold L * n_blocks entries and m_old n_blocks")
    st = lib().hkv_frame_headers(ctypes.byref(shape), FORMATS[fmt], ctypes.byref(fr),
                                 _i32(crc, "crc"), _i32(m_old, "m_old"), int(layer_base),
                                 _stream(stream, frames.device))
    _check("hkv_frame_headers", st)
    return frames


@_on_one_gpu
def frame_verify(frames, fmt, block_tokens: int, n_kv_heads: int, layer_base: int = 0,
                 out=None, stream=None):
    """Verification flags per frame: an int32 tensor [L, n_blocks] (0 = intact)."""
    shape, fr = _frame_args(frames, fmt, block_tokens, n_kv_heads)
    L, nb = frames.shape[0], frames.shape[1]
    if out is None:
        out = torch.empty((L, nb), dtype=torch.int32, device=frames.device)
    if out.numel() != L * nb:
        raise ValueError("out must hold L * n_blocks entries")
    st = lib().hkv_frame_verify(ctypes.byref(shape), FORMATS[fmt], ctypes.byref(fr),
                                int(layer_base), _i32(out, "out"),
                                _stream(stream, frames.device))
    _check("hkv_frame_verify", st)
    return out


@_on_one_gpu
def frame_delta_m(frames, fmt, block_tokens: int, n_kv_heads: int, m_new, out=None,
                  stream=None):
    """Per-block delta m_new - m_old from the first layer's frame headers."""
    shape, fr = _frame_args(frames, fmt, block_tokens, n_kv_heads)
    nb = frames.shape[1]
    if out is None:
        out = torch.empty(nb, dtype=torch.int32, device=frames.device)
    if out.numel() != nb or m_new.numel() != nb:
        raise ValueError("m_new and out must hold n_blocks entries")
    st = lib().hkv_frame_delta_m(ctypes.byref(shape), FORMATS[fmt], ctypes.byref(fr),
                                 _i32(m_new, "m_new"), _i32(out, "out"),
                                 _stream(stream, frames.device))
    _check("hkv_frame_delta_m", st)
    return out


@_on_one_gpu
def stream_probe(src, dst, stream=None):
    """Measurement aid: read src (uint8, a multiple of 128 bytes) and write it
    twice into dst (twice the size) with the fetch's store pattern."""
    if src.dtype != torch.uint8 or dst.dtype != torch.uint8:
        raise ValueError("src and dst must be uint8 tensors")
    if not src.is_contiguous() or not dst.is_contiguous() or dst.numel() < 2 * src.numel():
        raise ValueError("dst must be contiguous and hold twice src")
    _check("hkv_stream_probe", lib().hkv_stream_probe(
        ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), src.numel(),
        _stream(stream, src.device)))
    return dst


@_on_one_gpu
def stream_probe_put(src, dst, stream=None):
    """Measurement aid: read src (uint8, twice the size of dst) and write dst
    (a multiple of 128 bytes) with the put's load and store pattern."""
    if src.dtype != torch.uint8 or dst.dtype != torch.uint8:
        raise ValueError("src and dst must be uint8 tensors")
    if not src.is_contiguous() or not dst.is_contiguous() or src.numel() < 2 * dst.numel():
        raise ValueError("src must be contiguous and hold twice dst")
    _check("hkv_stream_probe_put", lib().hkv_stream_probe_put(
        ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), dst.numel(),
        _stream(stream, src.device)))
    return dst
