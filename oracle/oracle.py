"""ctypes wrapper around the plain C oracle of the lossless BF16 exponent codec.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline
leg may import this module; the product path never does.  It shares nothing with the
HIP library.  See zipccl_oracle.c for the format and the method citations
("ZipCCL ..." gist.science explanation page, sections 2.A-2.D).

Parity status of each function (how it is pinned, in tests/test_oracle_pins.py):
  plan_sigma            pinned: brute-force BF16 histogram of seeded Gaussian samples,
                        analytic coverage above 97 %, scale invariance sigma -> 2 sigma.
  plan_table            pinned: validation rules, ascending order.
  sample_sigma          pinned: a hand-computed sample (stride, Inf/NaN skipped, short
                        last tile), numpy fp64 root mean square of the same sample,
                        empty / all-NaN / all-zero segments give 1.
  compress / batch      pinned: hand-derived worked example (tests/golden), exhaustive
                        65 536-pattern round trip, size = 11 bits/value + escapes +
                        metadata, escape count = brute-force count, planted mistakes.
  decompress            pinned: exhaustive round trip (identity), corrupt-input errors.
  decompress_accumulate pinned: torch CPU fp32 sum rounded to BF16, subnormal and tie
                        cases, NaN rule.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "zipccl_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libzipccl_oracle.so")

OK, ERR_INVALID, ERR_SIZE, ERR_CORRUPT, ERR_OVERFLOW = 0, 1, 3, 5, 7

_c_u8p = ctypes.POINTER(ctypes.c_uint8)
_c_u16p = ctypes.POINTER(ctypes.c_uint16)
_c_u64p = ctypes.POINTER(ctypes.c_uint64)


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc: strict IEEE (no fast-math, no contraction)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str = _LIB_PATH, src: str = _SRC) -> ctypes.CDLL:
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(src):
        build(src=src, out=path)
    lib = ctypes.CDLL(path)
    lib.zo_static_size.restype = ctypes.c_uint64
    lib.zo_static_size.argtypes = [ctypes.c_uint64]
    lib.zo_binade_mass.restype = ctypes.c_double
    lib.zo_binade_mass.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.zo_plan_sigma.restype = ctypes.c_int
    lib.zo_plan_sigma.argtypes = [ctypes.c_double, _c_u8p]
    lib.zo_sample_sigma.restype = ctypes.c_double
    lib.zo_sample_sigma.argtypes = [_c_u16p, ctypes.c_uint64, ctypes.c_uint64]
    lib.zo_plan_table.restype = ctypes.c_int
    lib.zo_plan_table.argtypes = [_c_u8p, _c_u8p]
    lib.zo_compress.restype = ctypes.c_int
    lib.zo_compress.argtypes = [_c_u16p, ctypes.c_uint64, _c_u8p, ctypes.c_uint64, _c_u8p, _c_u8p,
                                ctypes.c_uint64, _c_u64p]
    lib.zo_compress_batch.restype = ctypes.c_int
    lib.zo_compress_batch.argtypes = [ctypes.c_int, ctypes.POINTER(_c_u16p), _c_u64p, _c_u8p, _c_u8p,
                                      _c_u8p, ctypes.c_uint64, _c_u64p]
    lib.zo_decompress.restype = ctypes.c_int
    lib.zo_decompress.argtypes = [_c_u8p, ctypes.c_uint64, _c_u8p, ctypes.c_uint64, ctypes.c_uint64,
                                  _c_u16p]
    lib.zo_decompress_accumulate.restype = ctypes.c_int
    lib.zo_decompress_accumulate.argtypes = [ctypes.c_int, ctypes.POINTER(_c_u8p), _c_u64p,
                                             ctypes.POINTER(_c_u8p), _c_u64p, ctypes.c_uint64,
                                             _c_u16p, _c_u16p]
    lib.zo_add2_bf16.restype = ctypes.c_uint16
    lib.zo_add2_bf16.argtypes = [ctypes.c_uint16, ctypes.c_uint16]
    lib.zo_round_bits.restype = ctypes.c_uint16
    lib.zo_round_bits.argtypes = [ctypes.c_uint32]
    return lib


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = load()
    return _lib


def use(handle: ctypes.CDLL) -> ctypes.CDLL:
    """Swap the loaded library (the planted-mistake tests load mutated copies)."""
    global _lib
    old, _lib = _lib, handle
    return old


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what} failed with code {code}")
        self.code = code


def _u8(a: np.ndarray):
    return a.ctypes.data_as(_c_u8p)


def _u16(a: np.ndarray):
    return a.ctypes.data_as(_c_u16p)


def _as_u16(x) -> np.ndarray:
    a = np.ascontiguousarray(x)
    if a.dtype != np.uint16:
        a = a.view(np.uint16) if a.dtype.itemsize == 2 else a.astype(np.uint16)
    return a


def static_size(n: int) -> int:
    return int(lib().zo_static_size(n))


def binade_mass(e: int, sigma: float) -> float:
    return float(lib().zo_binade_mass(e, sigma))


def plan_sigma(sigma: float) -> np.ndarray:
    t = np.zeros(7, np.uint8)
    rc = lib().zo_plan_sigma(float(sigma), _u8(t))
    if rc:
        raise OracleError(rc, "plan_sigma")
    return t


def sample_sigma(x, stride: int) -> float:
    """sigma of the finite values among tiles 0, stride, 2*stride, ... of 512 values."""
    x = _as_u16(x).ravel()
    buf = x if x.size else np.zeros(1, np.uint16)
    return float(lib().zo_sample_sigma(_u16(buf), x.size, stride))


def plan_table(table) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(table, dtype=np.uint8))
    if a.size != 7:
        raise OracleError(ERR_INVALID, "plan_table")
    t = np.zeros(7, np.uint8)
    rc = lib().zo_plan_table(_u8(a), _u8(t))
    if rc:
        raise OracleError(rc, "plan_table")
    return t


def compress(x, table, esc_offset: int = 0, esc=None, esc_cap=None):
    """One segment.  Returns (static bytes, escape bytes of this segment, n_esc)."""
    x = _as_u16(x).ravel()
    n = x.size
    t = np.ascontiguousarray(np.asarray(table, dtype=np.uint8))
    st = np.empty(static_size(n), np.uint8)
    own = esc is None
    if own:
        esc = np.zeros(max(esc_offset + n, 1), np.uint8)
        esc_cap = esc.size
    ne = ctypes.c_uint64(0)
    rc = lib().zo_compress(_u16(x), n, _u8(t), esc_offset, _u8(st), _u8(esc), esc_cap, ctypes.byref(ne))
    if rc not in (OK, ERR_OVERFLOW):
        raise OracleError(rc, "compress")
    k = int(ne.value)
    return st, (esc[esc_offset:esc_offset + k].copy() if own else None), k


def compress_batch(xs, tables, esc_cap=None):
    """Several segments in one call.  Returns (static bytes, escapes, n_esc list, rc)."""
    xs = [_as_u16(x).ravel() for x in xs]
    nseg = len(xs)
    ns = np.array([x.size for x in xs], np.uint64)
    tabs = np.ascontiguousarray(np.asarray(tables, dtype=np.uint8).reshape(nseg, 7))
    total_static = sum(static_size(int(n)) for n in ns)
    st = np.empty(total_static, np.uint8)
    if esc_cap is None:
        esc_cap = int(ns.sum())
    esc = np.zeros(max(esc_cap, 1), np.uint8)
    ptrs = (_c_u16p * max(nseg, 1))(*[_u16(x) for x in xs])
    ne = np.zeros(max(nseg, 1), np.uint64)
    rc = lib().zo_compress_batch(nseg, ptrs, ns.ctypes.data_as(_c_u64p), _u8(tabs), _u8(st), _u8(esc),
                                 esc_cap, ne.ctypes.data_as(_c_u64p))
    if rc not in (OK, ERR_OVERFLOW):
        raise OracleError(rc, "compress_batch")
    ne = ne[:nseg]
    used = min(int(ne.sum()), esc_cap)
    return st, esc[:used].copy(), [int(v) for v in ne], rc


def decompress(st, esc, n: int) -> np.ndarray:
    st = np.ascontiguousarray(st, dtype=np.uint8)
    esc = np.ascontiguousarray(esc, dtype=np.uint8)
    if esc.size == 0:
        esc = np.zeros(1, np.uint8)
        esc_bytes = 0
    else:
        esc_bytes = esc.size
    out = np.empty(max(n, 1), np.uint16)
    rc = lib().zo_decompress(_u8(st), st.size, _u8(esc), esc_bytes, n, _u16(out))
    if rc:
        raise OracleError(rc, "decompress")
    return out[:n]


def decompress_accumulate(sts, escs, n: int, local) -> np.ndarray:
    P = len(sts)
    sts = [np.ascontiguousarray(s, dtype=np.uint8) for s in sts]
    escs = [np.ascontiguousarray(e, dtype=np.uint8) for e in escs]
    esc_sizes = np.array([e.size for e in escs], np.uint64)
    escs = [e if e.size else np.zeros(1, np.uint8) for e in escs]
    st_sizes = np.array([s.size for s in sts], np.uint64)
    local = _as_u16(local).ravel()
    out = np.empty(max(n, 1), np.uint16)
    sp = (_c_u8p * max(P, 1))(*[_u8(s) for s in sts])
    ep = (_c_u8p * max(P, 1))(*[_u8(e) for e in escs])
    rc = lib().zo_decompress_accumulate(P, sp, st_sizes.ctypes.data_as(_c_u64p), ep,
                                        esc_sizes.ctypes.data_as(_c_u64p), n, _u16(local), _u16(out))
    if rc:
        raise OracleError(rc, "decompress_accumulate")
    return out[:n]


def add2_bf16(a: int, b: int) -> int:
    return int(lib().zo_add2_bf16(a, b))


def round_bits(f32bits: int) -> int:
    return int(lib().zo_round_bits(f32bits))
