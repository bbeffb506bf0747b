"""Python binding of libzipccl (ctypes).  Argument marshalling only: every step of the
codec runs in the library's HIP kernels; torch supplies device memory and streams.

The names mirror the C ABI in include/zipccl.h.  There is no CPU fallback: if the
library is not built, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libzipccl.so")

OK, ERR_INVALID, ERR_ALIGN, ERR_SIZE, ERR_HIP, ERR_CORRUPT = range(6)
STATUS_ESC_OVERFLOW, STATUS_CORRUPT, STATUS_BAD_INDEX, STATUS_WAIT_LIMIT = 1, 2, 4, 8
MAX_SEGMENTS, MAX_PEERS = 64, 16
FORMAT_VERSION, MAGIC = 1, 0x3143435A


class PlanT(ctypes.Structure):
    _fields_ = [("table", ctypes.c_uint8 * 7), ("reserved", ctypes.c_uint8)]

    @property
    def exponents(self):
        return list(self.table)

    def __repr__(self):
        return f"Plan({list(self.table)})"


class SegmentT(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("n", ctypes.c_uint64), ("plan", PlanT)]


class GatherSegmentT(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("src_rows", ctypes.c_uint64), ("row_len", ctypes.c_uint64),
                ("rows", ctypes.c_void_p), ("nrows", ctypes.c_uint64), ("plan", PlanT)]


class CodecProfileT(ctypes.Structure):
    _fields_ = [("compress_GBps", ctypes.c_double), ("accumulate_GBps", ctypes.c_double),
                ("compressed_fraction", ctypes.c_double)]


class LinkT(ctypes.Structure):
    _fields_ = [("bw_GBps", ctypes.c_double), ("latency_us", ctypes.c_double), ("links", ctypes.c_int)]


class DSegmentT(ctypes.Structure):
    _fields_ = [("dst", ctypes.c_void_p), ("n", ctypes.c_uint64)]


class ZipcclError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = _lib.zipccl_strerror(status).decode() if _lib is not None else str(status)
        super().__init__(f"{what}: {msg} (status {status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python -m lossless_bf16_exponent_codec_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    vp, u64, i32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int
    lib.zipccl_strerror.restype = ctypes.c_char_p
    lib.zipccl_strerror.argtypes = [i32]
    lib.zipccl_plan.restype = i32
    lib.zipccl_plan.argtypes = [ctypes.c_double, ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(PlanT)]
    lib.zipccl_plan_many.restype = i32
    lib.zipccl_plan_many.argtypes = [ctypes.POINTER(ctypes.c_double), i32, ctypes.POINTER(PlanT)]
    lib.zipccl_static_size.restype = u64
    lib.zipccl_static_size.argtypes = [u64]
    lib.zipccl_compressed_size.restype = u64
    lib.zipccl_compressed_size.argtypes = [u64, u64]
    lib.zipccl_workspace_size.restype = u64
    lib.zipccl_workspace_size.argtypes = [u64, i32]
    lib.zipccl_compress.restype = i32
    lib.zipccl_compress.argtypes = [ctypes.POINTER(SegmentT), i32, vp, u64, vp, u64, vp, u64, vp, vp, vp]
    lib.zipccl_compress_noalloc.restype = i32
    lib.zipccl_compress_noalloc.argtypes = [ctypes.POINTER(SegmentT), i32, vp, u64, vp, u64, vp, vp, vp]
    lib.zipccl_compress_chunks.restype = i32
    lib.zipccl_compress_chunks.argtypes = [ctypes.POINTER(SegmentT), i32, i32, ctypes.POINTER(vp),
                                           ctypes.POINTER(u64), ctypes.POINTER(vp), ctypes.POINTER(u64), vp, u64,
                                           vp, vp, vp]
    lib.zipccl_estimate_plans.restype = i32
    lib.zipccl_estimate_plans.argtypes = [ctypes.POINTER(SegmentT), i32, ctypes.c_uint32, vp, vp, u64, vp]
    lib.zipccl_estimate_workspace_size.restype = u64
    lib.zipccl_estimate_workspace_size.argtypes = [i32]
    lib.zipccl_compress_device_plans.restype = i32
    lib.zipccl_compress_device_plans.argtypes = [ctypes.POINTER(SegmentT), i32, vp, vp, u64, vp, u64, vp, u64, vp,
                                                 vp, vp]
    lib.zipccl_compress_gather.restype = i32
    lib.zipccl_compress_gather.argtypes = [ctypes.POINTER(GatherSegmentT), i32, vp, u64, vp, u64, vp, u64, vp, vp,
                                           vp]
    lib.zipccl_decompress.restype = i32
    lib.zipccl_decompress.argtypes = [vp, u64, vp, u64, ctypes.POINTER(DSegmentT), i32, vp, vp]
    lib.zipccl_decompress_shards.restype = i32
    lib.zipccl_decompress_shards.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(u64),
                                             ctypes.POINTER(DSegmentT), i32, ctypes.c_uint32, vp, vp]
    lib.zipccl_decompress_accumulate.restype = i32
    lib.zipccl_decompress_accumulate.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(u64), i32,
                                                 u64, vp, vp, vp, vp]
    lib.zipccl_decompress_accumulate_chunks.restype = i32
    lib.zipccl_decompress_accumulate_chunks.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(u64),
                                                        i32, u64, u64, vp, vp, vp, vp]
    lib.zipccl_profile_scratch_size.restype = u64
    lib.zipccl_profile_scratch_size.argtypes = [u64, i32]
    lib.zipccl_profile_codec.restype = i32
    lib.zipccl_profile_codec.argtypes = [vp, u64, PlanT, i32, vp, u64, vp, ctypes.POINTER(CodecProfileT)]
    lib.zipccl_rs_choose.restype = i32
    lib.zipccl_rs_choose.argtypes = [ctypes.POINTER(CodecProfileT), ctypes.POINTER(LinkT), i32, u64,
                                     ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_double)]
    lib.zipccl_pipeline_scratch_size.restype = u64
    lib.zipccl_pipeline_scratch_size.argtypes = [i32, u64]
    lib.zipccl_pipeline_create.restype = i32
    lib.zipccl_pipeline_create.argtypes = [i32, u64, vp, u64, vp, vp, ctypes.POINTER(vp)]
    lib.zipccl_pipeline_reduce.restype = i32
    lib.zipccl_pipeline_reduce.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(PlanT), u64, vp, vp, vp]
    lib.zipccl_pipeline_destroy.restype = None
    lib.zipccl_pipeline_destroy.argtypes = [vp]
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def _check(rc: int, what: str):
    if rc != OK:
        raise ZipcclError(rc, what)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


# ------------------------------------------------------------------------------------
# C ABI mirrors
# ------------------------------------------------------------------------------------
def plan(sigma: float | None = None, table=None) -> PlanT:
    """zipccl_plan: sigma -> 7-exponent window, or a given table (sorted)."""
    out = PlanT()
    if table is not None:
        arr = (ctypes.c_uint8 * 7)(*[int(v) for v in table]) if len(table) == 7 else None
        if arr is None:
            raise ZipcclError(ERR_INVALID, "zipccl_plan")
        _check(_lib.zipccl_plan(0.0, arr, ctypes.byref(out)), "zipccl_plan")
    else:
        _check(_lib.zipccl_plan(float(sigma), None, ctypes.byref(out)), "zipccl_plan")
    return out


def plan_many(sigmas):
    """zipccl_plan_many: one plan per sigma, as a ctypes array of PlanT."""
    n = len(sigmas)
    sig = (ctypes.c_double * max(n, 1))(*[float(x) for x in sigmas])
    out = (PlanT * max(n, 1))()
    _check(_lib.zipccl_plan_many(sig, n, out), "zipccl_plan_many")
    return out


def static_size(n: int) -> int:
    return int(_lib.zipccl_static_size(n))


def compressed_size(n: int, n_esc: int) -> int:
    return int(_lib.zipccl_compressed_size(n, n_esc))


def workspace_size(total_n: int, nseg: int) -> int:
    return int(_lib.zipccl_workspace_size(total_n, nseg))


def compress(segments, static_out, esc_out, workspace, n_esc_out=None, status=None, stream=None,
             esc_cap: int | None = None):
    """zipccl_compress.  segments: list of (bf16 device tensor, PlanT)."""
    nseg = len(segments)
    arr = (SegmentT * max(nseg, 1))()
    for k, (t, p) in enumerate(segments):
        arr[k].src = _ptr(t) if t.numel() else None
        arr[k].n = t.numel()
        arr[k].plan = p
    cap = _nbytes(esc_out) if esc_cap is None else esc_cap
    rc = _lib.zipccl_compress(arr, nseg, _ptr(static_out), _nbytes(static_out), _ptr(esc_out), cap,
                              _ptr(workspace), _nbytes(workspace), _ptr(n_esc_out), _ptr(status), _stream(stream))
    _check(rc, "zipccl_compress")


NOALLOC_MAX_VALUES = 1 << 26


def compress_noalloc(segments, static_out, esc_out, n_esc_out=None, status=None, stream=None,
                     esc_cap: int | None = None):
    """zipccl_compress_noalloc: zipccl_compress with the library's static device workspace."""
    nseg = len(segments)
    arr = (SegmentT * max(nseg, 1))()
    for k, (t, p) in enumerate(segments):
        arr[k].src = _ptr(t) if t.numel() else None
        arr[k].n = t.numel()
        arr[k].plan = p
    cap = _nbytes(esc_out) if esc_cap is None else esc_cap
    rc = _lib.zipccl_compress_noalloc(arr, nseg, _ptr(static_out), _nbytes(static_out), _ptr(esc_out), cap,
                                      _ptr(n_esc_out), _ptr(status), _stream(stream))
    _check(rc, "zipccl_compress_noalloc")


class PreparedCompressChunks:
    """A zipccl_compress_chunks call over fixed buffers, marshalled once.  chunks: a list
    of per-chunk lists of bf16 device tensors (the same number in each); static_outs /
    esc_outs: per-chunk uint8 device tensors.  run(plans) uses plans[i] for segment i of
    every chunk.  esc_caps: per-chunk escape capacities (default: each buffer's size)."""

    def __init__(self, chunks, static_outs, esc_outs, workspace, n_esc_out=None, status=None, stream=None,
                 esc_caps=None):
        self.nchunks, self.nseg = len(chunks), len(chunks[0])
        self._arr = (SegmentT * (self.nchunks * self.nseg))()
        for k, tensors in enumerate(chunks):
            if len(tensors) != self.nseg:
                raise ValueError("every chunk needs the same number of segments")
            for i, t in enumerate(tensors):
                e = self._arr[k * self.nseg + i]
                e.src = _ptr(t) if t.numel() else None
                e.n = t.numel()
        C = self.nchunks
        sp = (ctypes.c_void_p * C)(*[_ptr(t) for t in static_outs])
        sc = (ctypes.c_uint64 * C)(*[_nbytes(t) for t in static_outs])
        ep = (ctypes.c_void_p * C)(*[_ptr(t) for t in esc_outs])
        ec = (ctypes.c_uint64 * C)(*([_nbytes(t) for t in esc_outs] if esc_caps is None else esc_caps))
        self._args = (sp, sc, ep, ec, _ptr(workspace), _nbytes(workspace), _ptr(n_esc_out), _ptr(status),
                      _stream(stream))
        self._keep = (chunks, static_outs, esc_outs, workspace, n_esc_out, status)

    def run(self, plans):
        for k in range(self.nchunks):
            for i in range(self.nseg):
                self._arr[k * self.nseg + i].plan = plans[i]
        _check(_lib.zipccl_compress_chunks(self._arr, self.nseg, self.nchunks, *self._args), "zipccl_compress_chunks")


def _segment_array(tensors):
    arr = (SegmentT * max(len(tensors), 1))()
    for k, t in enumerate(tensors):
        arr[k].src = _ptr(t) if t.numel() else None
        arr[k].n = t.numel()
    return arr


def estimate_workspace_size(nseg: int) -> int:
    return int(_lib.zipccl_estimate_workspace_size(nseg))


def estimate_plans(tensors, plans_dev, workspace, stride: int = 16, stream=None):
    """zipccl_estimate_plans: plans_dev, a uint8 device tensor of 8 * len(tensors) bytes,
    receives one plan per bf16 tensor (PlanT.from_buffer_copy on its bytes reads them);
    workspace, a device tensor of at least estimate_workspace_size(len(tensors)) bytes."""
    _check(_lib.zipccl_estimate_plans(_segment_array(tensors), len(tensors), stride, _ptr(plans_dev),
                                      _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "zipccl_estimate_plans")


def compress_device_plans(tensors, plans_dev, static_out, esc_out, workspace, n_esc_out=None, status=None,
                          stream=None, esc_cap: int | None = None):
    """zipccl_compress_device_plans: tensors coded by the plans in plans_dev (device)."""
    cap = _nbytes(esc_out) if esc_cap is None else esc_cap
    _check(_lib.zipccl_compress_device_plans(_segment_array(tensors), len(tensors), _ptr(plans_dev),
                                             _ptr(static_out), _nbytes(static_out), _ptr(esc_out), cap,
                                             _ptr(workspace), _nbytes(workspace), _ptr(n_esc_out), _ptr(status),
                                             _stream(stream)), "zipccl_compress_device_plans")


def compress_gather(segments, static_out, esc_out, workspace, n_esc_out=None, status=None, stream=None,
                    esc_cap: int | None = None):
    """zipccl_compress_gather.  segments: list of (matrix, rows, plan): matrix a 2-D bf16
    device tensor (row-major, contiguous), rows a 1-D int32 device tensor of row indices."""
    PreparedCompressGather(segments, static_out, esc_out, workspace, n_esc_out, status, stream, esc_cap).run()


class PreparedCompressGather:
    """A zipccl_compress_gather call over fixed buffers, marshalled once; run([plans])
    makes it."""

    def __init__(self, segments, static_out, esc_out, workspace, n_esc_out=None, status=None, stream=None,
                 esc_cap: int | None = None):
        nseg = len(segments)
        self._arr = (GatherSegmentT * max(nseg, 1))()
        for k, (m, rows, p) in enumerate(segments):
            if m.dim() != 2 or not m.is_contiguous() or rows.dtype != torch.int32:
                raise ValueError("compress_gather takes a contiguous 2-D matrix and int32 row indices")
            self._arr[k].src = _ptr(m) if m.numel() else None
            self._arr[k].src_rows = m.shape[0]
            self._arr[k].row_len = m.shape[1]
            self._arr[k].rows = _ptr(rows) if rows.numel() else None
            self._arr[k].nrows = rows.numel()
            self._arr[k].plan = p
        cap = _nbytes(esc_out) if esc_cap is None else esc_cap
        self._args = (self._arr, nseg, _ptr(static_out), _nbytes(static_out), _ptr(esc_out), cap, _ptr(workspace),
                      _nbytes(workspace), _ptr(n_esc_out), _ptr(status), _stream(stream))
        self._keep = (segments, static_out, esc_out, workspace, n_esc_out, status)

    def run(self, plans=None):
        """Makes the call; `plans`, if given, replaces the segments' plans first."""
        if plans is not None:
            for k, p in enumerate(plans):
                self._arr[k].plan = p
        _check(_lib.zipccl_compress_gather(*self._args), "zipccl_compress_gather")


def decompress(static_in, esc_in, dsts, status=None, stream=None, static_bytes=None, esc_bytes=None):
    """zipccl_decompress.  dsts: list of bf16 device tensors (their numel is n)."""
    nseg = len(dsts)
    arr = (DSegmentT * max(nseg, 1))()
    for k, t in enumerate(dsts):
        arr[k].dst = _ptr(t) if t.numel() else None
        arr[k].n = t.numel()
    sb = _nbytes(static_in) if static_bytes is None else static_bytes
    eb = (_nbytes(esc_in) if esc_in is not None else 0) if esc_bytes is None else esc_bytes
    rc = _lib.zipccl_decompress(_ptr(static_in), sb, _ptr(esc_in), eb, arr, nseg, _ptr(status), _stream(stream))
    _check(rc, "zipccl_decompress")


SHARDS_ESC_AT_FIRST = 1


def decompress_shards(static_ins, esc_ins, dsts, status=None, stream=None, esc_bytes=None, flags=0):
    """zipccl_decompress_shards.  static_ins / esc_ins: per-shard device tensors or raw
    device addresses (int; an escape entry may be None); dsts: bf16 device tensors, one
    per shard (their numel is n); esc_bytes: per-shard escape buffer sizes; flags:
    SHARDS_ESC_AT_FIRST when each escape buffer starts at its shard's first escape."""
    PreparedDecompressShards(static_ins, esc_ins, dsts, status, stream, esc_bytes, flags).run()


class PreparedDecompressShards:
    """A zipccl_decompress_shards call over fixed buffers, marshalled once; run() makes it."""

    def __init__(self, static_ins, esc_ins, dsts, status=None, stream=None, esc_bytes=None, flags=0):
        nseg = len(dsts)
        sp = (ctypes.c_void_p * nseg)(*[_ptr(t) for t in static_ins])
        ep = (ctypes.c_void_p * nseg)(*[_ptr(t) for t in esc_ins])
        if esc_bytes is None:
            esc_bytes = [_nbytes(t) if t is not None else 0 for t in esc_ins]
        eb = (ctypes.c_uint64 * nseg)(*[int(v) for v in esc_bytes])
        arr = (DSegmentT * max(nseg, 1))()
        for k, t in enumerate(dsts):
            arr[k].dst = _ptr(t) if t.numel() else None
            arr[k].n = t.numel()
        self._args = (sp, ep, eb, arr, nseg, flags, _ptr(status), _stream(stream))
        self._keep = (static_ins, esc_ins, dsts, status)

    def run(self):
        _check(_lib.zipccl_decompress_shards(*self._args), "zipccl_decompress_shards")


def decompress_accumulate(static_ins, esc_ins, n: int, local, dst, status=None, stream=None, esc_bytes=None):
    """zipccl_decompress_accumulate.  static_ins / esc_ins: per-peer device tensors or
    raw device addresses (int); esc_bytes: per-peer escape buffer sizes."""
    P = len(static_ins)
    sp = (ctypes.c_void_p * P)(*[_ptr(t) for t in static_ins])
    ep = (ctypes.c_void_p * P)(*[_ptr(t) for t in esc_ins])
    if esc_bytes is None:
        esc_bytes = [_nbytes(t) for t in esc_ins]
    eb = (ctypes.c_uint64 * P)(*[int(v) for v in esc_bytes])
    rc = _lib.zipccl_decompress_accumulate(sp, ep, eb, P, n, _ptr(local), _ptr(dst), _ptr(status), _stream(stream))
    _check(rc, "zipccl_decompress_accumulate")


class PreparedCompress:
    """A zipccl_compress call over fixed buffers: the segment table and every other
    argument are marshalled once; run(plans) writes this call's plans into the table and
    makes the call (for loops that compress the same buffers with new plans)."""

    def __init__(self, tensors, static_out, esc_out, workspace, n_esc_out=None, status=None, stream=None,
                 esc_cap=None):
        self.n = len(tensors)
        self._arr = (SegmentT * max(self.n, 1))()
        for k, t in enumerate(tensors):
            self._arr[k].src = _ptr(t) if t.numel() else None
            self._arr[k].n = t.numel()
        cap = _nbytes(esc_out) if esc_cap is None else esc_cap
        self._args = (_ptr(static_out), _nbytes(static_out), _ptr(esc_out), cap, _ptr(workspace),
                      _nbytes(workspace), _ptr(n_esc_out), _ptr(status), _stream(stream))
        self._keep = (tensors, static_out, esc_out, workspace, n_esc_out, status)

    def run(self, plans):
        arr = self._arr
        for k in range(self.n):
            arr[k].plan = plans[k]
        _check(_lib.zipccl_compress(arr, self.n, *self._args), "zipccl_compress")


class PreparedDecompress:
    """A zipccl_decompress call over fixed buffers, marshalled once; run() makes it."""

    def __init__(self, static_in, esc_in, dsts, status=None, stream=None, static_bytes=None, esc_bytes=None):
        self.n = len(dsts)
        self._arr = (DSegmentT * max(self.n, 1))()
        for k, t in enumerate(dsts):
            self._arr[k].dst = _ptr(t) if t.numel() else None
            self._arr[k].n = t.numel()
        sb = _nbytes(static_in) if static_bytes is None else static_bytes
        eb = (_nbytes(esc_in) if esc_in is not None else 0) if esc_bytes is None else esc_bytes
        self._args = (_ptr(static_in), sb, _ptr(esc_in), eb, self._arr, self.n, _ptr(status), _stream(stream))
        self._keep = (static_in, esc_in, dsts, status)

    def run(self):
        _check(_lib.zipccl_decompress(*self._args), "zipccl_decompress")


class PreparedAccumulate:
    """A zipccl_decompress_accumulate call over fixed buffers, marshalled once."""

    def __init__(self, static_ins, esc_ins, n: int, local, dst, status=None, stream=None, esc_bytes=None):
        P = len(static_ins)
        self._sp = (ctypes.c_void_p * P)(*[_ptr(t) for t in static_ins])
        self._ep = (ctypes.c_void_p * P)(*[_ptr(t) for t in esc_ins])
        if esc_bytes is None:
            esc_bytes = [_nbytes(t) for t in esc_ins]
        self._eb = (ctypes.c_uint64 * P)(*[int(v) for v in esc_bytes])
        self._args = (self._sp, self._ep, self._eb, P, n, _ptr(local), _ptr(dst), _ptr(status), _stream(stream))
        self._keep = (static_ins, esc_ins, local, dst, status)

    def run(self):
        _check(_lib.zipccl_decompress_accumulate(*self._args), "zipccl_decompress_accumulate")


def pipeline_scratch_size(npeers: int, chunk: int) -> int:
    return int(_lib.zipccl_pipeline_scratch_size(npeers, chunk))


class PreparedAccumulateChunks:
    """A zipccl_decompress_accumulate_chunks call over fixed buffers, marshalled once.
    static_ins / esc_ins / esc_bytes: per-(chunk, peer) entries, chunk-major (device
    tensors or raw addresses); n values of local and dst in chunks of `chunk`."""

    def __init__(self, static_ins, esc_ins, npeers: int, chunk: int, n: int, local, dst, status=None,
                 stream=None, esc_bytes=None):
        m = len(static_ins)
        sp = (ctypes.c_void_p * m)(*[_ptr(t) for t in static_ins])
        ep = (ctypes.c_void_p * m)(*[_ptr(t) for t in esc_ins])
        if esc_bytes is None:
            esc_bytes = [_nbytes(t) for t in esc_ins]
        eb = (ctypes.c_uint64 * m)(*[int(v) for v in esc_bytes])
        self._args = (sp, ep, eb, npeers, chunk, n, _ptr(local), _ptr(dst), _ptr(status), _stream(stream))
        self._keep = (static_ins, esc_ins, local, dst, status)

    def run(self):
        _check(_lib.zipccl_decompress_accumulate_chunks(*self._args), "zipccl_decompress_accumulate_chunks")


def profile_codec(sample, plan, npeers: int, stream=None) -> CodecProfileT:
    """zipccl_profile_codec on a bf16 device tensor (scratch allocated with torch)."""
    n = sample.numel()
    size = _lib.zipccl_profile_scratch_size(n, npeers)
    scratch = torch.empty(max(size, 1), dtype=torch.uint8, device=sample.device)
    out = CodecProfileT()
    _check(_lib.zipccl_profile_codec(_ptr(sample), n, plan, npeers, _ptr(scratch), size, _stream(stream),
                                     ctypes.byref(out)), "zipccl_profile_codec")
    return out


def rs_choose(profile: CodecProfileT, link: LinkT, ranks: int, nbytes: int):
    """zipccl_rs_choose: (use_codec, native_us, zipped_us)."""
    use = ctypes.c_int32()
    t_n, t_z = ctypes.c_double(), ctypes.c_double()
    _check(_lib.zipccl_rs_choose(ctypes.byref(profile), ctypes.byref(link), ranks, nbytes, ctypes.byref(use),
                                 ctypes.byref(t_n), ctypes.byref(t_z)), "zipccl_rs_choose")
    return bool(use.value), t_n.value, t_z.value


class Pipeline:
    """zipccl_pipeline_*: chunked compress (stream_a) -> decode-accumulate (stream_b)."""

    def __init__(self, npeers: int, chunk: int, stream_a, stream_b, device=None):
        self.npeers, self.chunk = npeers, chunk
        size = pipeline_scratch_size(npeers, chunk)
        self.scratch = torch.zeros(size, dtype=torch.uint8, device=device or "cuda")
        h = ctypes.c_void_p()
        rc = _lib.zipccl_pipeline_create(npeers, chunk, _ptr(self.scratch), size, _stream(stream_a),
                                         _stream(stream_b), ctypes.byref(h))
        _check(rc, "zipccl_pipeline_create")
        self._h = h
        self.stream_a, self.stream_b = stream_a, stream_b

    def reduce(self, peer_src, plans, local, dst, status=None):
        P = self.npeers
        sp = (ctypes.c_void_p * P)(*[_ptr(t) for t in peer_src])
        pl = (PlanT * P)(*plans)
        rc = _lib.zipccl_pipeline_reduce(self._h, sp, pl, local.numel(), _ptr(local), _ptr(dst), _ptr(status))
        _check(rc, "zipccl_pipeline_reduce")

    def close(self):
        # at interpreter exit the module globals may already be gone
        if getattr(self, "_h", None) and _lib is not None:
            _lib.zipccl_pipeline_destroy(self._h)
        self._h = None

    def __del__(self):
        self.close()


# ------------------------------------------------------------------------------------
# convenience: buffers from torch, one call each way
# ------------------------------------------------------------------------------------
@dataclass
class Compressed:
    static: torch.Tensor        # uint8, segments back to back
    esc: torch.Tensor           # uint8, escape capacity
    n_esc: torch.Tensor         # uint64 as int64, nseg + 1 entries (last = total)
    sizes: list                 # n of each segment
    status: torch.Tensor        # int32 device status word

    def static_sizes(self):
        return [static_size(n) for n in self.sizes]


def _as_bf16(t):
    return t if t.dtype == torch.bfloat16 else t.view(torch.bfloat16)


def compress_tensors(tensors, plans, esc_cap=None, workspace=None, stream=None) -> Compressed:
    """Allocates outputs with torch and compresses the tensors in one launch."""
    dev = tensors[0].device
    sizes = [t.numel() for t in tensors]
    total_static = sum(static_size(n) for n in sizes)
    static = torch.empty(max(total_static, 1), dtype=torch.uint8, device=dev)
    cap = sum(sizes) if esc_cap is None else esc_cap
    esc = torch.empty(max(cap, 1), dtype=torch.uint8, device=dev)
    n_esc = torch.zeros(len(tensors) + 1, dtype=torch.int64, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(workspace_size(sum(sizes), len(tensors)), dtype=torch.uint8, device=dev)
    compress([(_as_bf16(t), p) for t, p in zip(tensors, plans)], static, esc, workspace, n_esc, status,
             stream=stream, esc_cap=cap)
    return Compressed(static, esc, n_esc, sizes, status)


def decompress_tensors(c: Compressed, out=None, stream=None):
    dev = c.static.device
    if out is None:
        out = [torch.empty(n, dtype=torch.bfloat16, device=dev) for n in c.sizes]
    decompress(c.static, c.esc, out, c.status, stream=stream)
    return out
