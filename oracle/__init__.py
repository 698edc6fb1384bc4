"""Plain CPU oracle of the chunked byte-plane + rANS weight codec.

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously-correct
definition that the GPU library is checked against.  Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it; the product
package never does, and it shares no code with it.

The arithmetic lives in ``wc_oracle.c`` (plain C, built with gcc); this module
only builds and loads that library and marshals numpy arrays.  The format it
defines is described at the top of ``wc_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wc_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libwc_oracle.so")

BF16, FP32, BF16_REORDER, FP16, FP16_REORDER, FP8_E4M3, FP8_E5M2 = 0, 1, 2, 3, 4, 5, 6
DTYPES = {"bf16": BF16, "fp32": FP32, "bf16r": BF16_REORDER, "fp16": FP16, "fp16r": FP16_REORDER,
          "fp8e4m3": FP8_E4M3, "fp8e5m2": FP8_E5M2}
# option bits of a format word
OPT_TENSOR_TABLE = 0x100  # one table per tensor
OPT_RAW_FALLBACK = 0x200  # chunks that do not shrink are stored raw
OPT_CRC32 = 0x400         # a CRC-32 of every chunk's payload

OK, ERR_ARG, ERR_CAPACITY, ERR_CORRUPT = 0, 1, 2, 3
EF_BAD_TABLE, EF_WORD_OVERRUN, EF_BAD_FINAL_STATE, EF_BAD_TAIL, EF_BAD_SEEK = 1, 2, 4, 8, 16
EF_BAD_CRC = 64

CHUNK = 65536


def build(force: bool = True) -> str:
    """Compile ``libwc_oracle.so`` next to its source with gcc."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread",
               _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Layout(ctypes.Structure):
    _fields_ = [("n", ctypes.c_uint64), ("num_chunks", ctypes.c_uint64),
                ("raw_bytes", ctypes.c_uint64), ("table_bytes", ctypes.c_uint64),
                ("seek_bytes", ctypes.c_uint64), ("payload_capacity", ctypes.c_uint64)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        P, U64, U32, I = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int
        L.wco_query_layout.argtypes = [I, U64, ctypes.POINTER(_Layout)]
        L.wco_split_bf16.argtypes = [P, U64, P, P]
        L.wco_merge_bf16.argtypes = [P, P, U64, P]
        L.wco_split_fp32.argtypes = [P, U64, P, P]
        L.wco_merge_fp32.argtypes = [P, P, U64, P]
        L.wco_histogram.argtypes = [P, U32, P]
        L.wco_normalize.argtypes = [P, U32, P]
        L.wco_normalize64.argtypes = [P, U64, P]
        L.wco_split_u16.argtypes = [I, P, U64, P, P]
        L.wco_split_fp8.argtypes = [I, P, U64, P, P]
        L.wco_crc32.argtypes = [P, U64]
        L.wco_crc32.restype = U32
        L.wco_chunk_crc.argtypes = [P, P, U64, P]
        L.wco_tile_order.argtypes = [P, P, U32, U32, I]
        L.wco_gemm_bf16.argtypes = [P, P, U32, U32, U32, P, P]
        L.wco_merge_fp8.argtypes = [I, P, P, U64, P]
        L.wco_merge_u16.argtypes = [I, P, P, U64, P]
        L.wco_encode_chunk.argtypes = [P, U32, P, P]
        L.wco_encode_chunk.restype = U32
        L.wco_decode_chunk.argtypes = [P, U64, P, U32, P]
        L.wco_decode_chunk.restype = U32
        L.wco_encode.argtypes = [I, P, U64, P, P, P, P, U64, I]
        L.wco_decode.argtypes = [I, P, P, P, P, U64, U64, P, I, ctypes.POINTER(U32)]
        L.wco_plan_batch.argtypes = [I, P, U32, P, P, ctypes.POINTER(_Layout)]
        L.wco_encode_batch.argtypes = [I, P, P, U32, P, P, P, P, U64, I]
        L.wco_decode_batch.argtypes = [I, P, P, U32, P, P, P, P, U64, I, ctypes.POINTER(U32)]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dt(dtype, options: int = 0) -> int:
    """Format word: the layout named by `dtype` OR-ed with option bits."""
    return (DTYPES[dtype] if isinstance(dtype, str) else int(dtype)) | int(options)


def options(tensor_table: bool = False, raw_fallback: bool = False) -> int:
    return (OPT_TENSOR_TABLE if tensor_table else 0) | (OPT_RAW_FALLBACK if raw_fallback else 0)


def elem_type(dtype):
    if dtype in ("fp32", FP32):
        return np.uint32
    if dtype in ("fp8e4m3", "fp8e5m2", FP8_E4M3, FP8_E5M2):
        return np.uint8
    return np.uint16


@dataclass
class Layout:
    n: int
    num_chunks: int
    raw_bytes: int
    table_bytes: int
    seek_bytes: int
    payload_capacity: int


def query_layout(dtype, n: int, opts: int = 0) -> Layout:
    out = _Layout()
    rc = lib().wco_query_layout(_dt(dtype, opts), n, ctypes.byref(out))
    if rc != OK:
        raise ValueError(f"wco_query_layout failed: {rc}")
    return Layout(out.n, out.num_chunks, out.raw_bytes, out.table_bytes, out.seek_bytes,
                  out.payload_capacity)


# ------------------------------------------------------------------ planes

def split_bf16(v: np.ndarray):
    v = np.ascontiguousarray(v, dtype=np.uint16).ravel()
    hi = np.empty(v.size, np.uint8)
    lo = np.empty(v.size, np.uint8)
    lib().wco_split_bf16(_p(v), v.size, _p(hi), _p(lo))
    return hi, lo


def merge_bf16(hi: np.ndarray, lo: np.ndarray) -> np.ndarray:
    hi = np.ascontiguousarray(hi, np.uint8)
    lo = np.ascontiguousarray(lo, np.uint8)
    v = np.empty(hi.size, np.uint16)
    lib().wco_merge_bf16(_p(hi), _p(lo), hi.size, _p(v))
    return v


def split_u16(layout, v: np.ndarray):
    """Any 16-bit layout ("bf16", "bf16r", "fp16", "fp16r"): (coded, raw)."""
    v = np.ascontiguousarray(v, dtype=np.uint16).ravel()
    hi = np.empty(v.size, np.uint8)
    lo = np.empty(v.size, np.uint8)
    lib().wco_split_u16(_dt(layout), _p(v), v.size, _p(hi), _p(lo))
    return hi, lo


def merge_u16(layout, hi: np.ndarray, lo: np.ndarray) -> np.ndarray:
    hi = np.ascontiguousarray(hi, np.uint8)
    lo = np.ascontiguousarray(lo, np.uint8)
    v = np.empty(hi.size, np.uint16)
    lib().wco_merge_u16(_dt(layout), _p(hi), _p(lo), hi.size, _p(v))
    return v


def split_fp8(layout, v: np.ndarray):
    """FP8 layouts ("fp8e4m3", "fp8e5m2"): (coded nibbles, packed raw nibbles)."""
    v = np.ascontiguousarray(v, dtype=np.uint8).ravel()
    coded = np.empty(v.size, np.uint8)
    raw = np.empty((v.size + 1) // 2, np.uint8)
    lib().wco_split_fp8(_dt(layout), _p(v), v.size, _p(coded), _p(raw))
    return coded, raw


def merge_fp8(layout, coded: np.ndarray, raw: np.ndarray) -> np.ndarray:
    coded = np.ascontiguousarray(coded, np.uint8)
    raw = np.ascontiguousarray(raw, np.uint8)
    v = np.empty(coded.size, np.uint8)
    lib().wco_merge_fp8(_dt(layout), _p(coded), _p(raw), coded.size, _p(v))
    return v


def split_fp32(u: np.ndarray):
    u = np.ascontiguousarray(u, dtype=np.uint32).ravel()
    exp = np.empty(u.size, np.uint8)
    raw = np.empty(query_layout("fp32", u.size).raw_bytes, np.uint8)
    lib().wco_split_fp32(_p(u), u.size, _p(exp), _p(raw))
    return exp, raw


def merge_fp32(exp: np.ndarray, raw: np.ndarray) -> np.ndarray:
    exp = np.ascontiguousarray(exp, np.uint8)
    raw = np.ascontiguousarray(raw, np.uint8)
    u = np.empty(exp.size, np.uint32)
    lib().wco_merge_fp32(_p(exp), _p(raw), exp.size, _p(u))
    return u


# ------------------------------------------------------------- one chunk

def histogram(sym: np.ndarray) -> np.ndarray:
    sym = np.ascontiguousarray(sym, np.uint8)
    c = np.empty(256, np.uint32)
    lib().wco_histogram(_p(sym), sym.size, _p(c))
    return c


def normalize(counts, total: int | None = None) -> np.ndarray:
    c = np.ascontiguousarray(counts, np.uint32)
    assert c.size == 256
    if total is None:
        total = int(c.sum())
    f = np.empty(256, np.uint16)
    lib().wco_normalize(_p(c), total, _p(f))
    return f


def normalize64(counts, total: int | None = None) -> np.ndarray:
    """The same normalisation for 64-bit counts (a whole tensor's histogram)."""
    c = np.ascontiguousarray(counts, np.uint64)
    assert c.size == 256
    if total is None:
        total = int(c.sum())
    f = np.empty(256, np.uint16)
    lib().wco_normalize64(_p(c), total, _p(f))
    return f


def encode_chunk(sym: np.ndarray, freq: np.ndarray) -> np.ndarray:
    sym = np.ascontiguousarray(sym, np.uint8)
    freq = np.ascontiguousarray(freq, np.uint16)
    assert 1 <= sym.size <= CHUNK
    out = np.zeros(128 + 2 * sym.size + 2, np.uint8)
    size = lib().wco_encode_chunk(_p(sym), sym.size, _p(freq), _p(out))
    return out[:size].copy()


def decode_chunk(payload: np.ndarray, freq: np.ndarray, n: int):
    payload = np.ascontiguousarray(payload, np.uint8)
    freq = np.ascontiguousarray(freq, np.uint16)
    sym = np.zeros(n, np.uint8)
    err = lib().wco_decode_chunk(_p(payload), payload.size, _p(freq), n, _p(sym))
    return sym, int(err)


# ------------------------------------------------------------------ CRC-32

def crc32(data) -> int:
    a = np.ascontiguousarray(np.frombuffer(bytes(data), np.uint8) if isinstance(data, (bytes, bytearray))
                             else data, np.uint8)
    buf = a if a.size else np.zeros(1, np.uint8)
    return int(lib().wco_crc32(_p(buf), a.size))


def chunk_crc(seek: np.ndarray, payload: np.ndarray) -> np.ndarray:
    """CRC-32 of every chunk's payload bytes."""
    seek = np.ascontiguousarray(seek, np.uint64)
    payload = np.ascontiguousarray(payload, np.uint8)
    pay = payload if payload.size else np.zeros(1, np.uint8)
    out = np.zeros(max(seek.size - 1, 1), np.uint32)
    lib().wco_chunk_crc(_p(seek), _p(pay), seek.size - 1, _p(out))
    return out[: seek.size - 1]


# -------------------------------------------------- tile order and GEMM

def tile_order(w: np.ndarray, inverse: bool = False, shape=None) -> np.ndarray:
    """The tile order of a rows x cols matrix of 16-bit patterns (flat
    result), or with inverse the matrix (shape = (rows, cols)) from its
    tile-ordered values.  Order defined in wc_oracle.c (wco_tile_order)."""
    if inverse:
        rows, cols = shape
        src = np.ascontiguousarray(w, np.uint16).reshape(-1)
    else:
        rows, cols = w.shape
        src = np.ascontiguousarray(w, np.uint16).reshape(-1)
    if src.size != rows * cols:
        raise ValueError("size does not match the shape")
    out = np.empty(rows * cols, np.uint16)
    if src.size:
        rc = lib().wco_tile_order(_p(src), _p(out), rows, cols, 1 if inverse else 0)
        if rc != OK:
            raise ValueError(f"tile order needs rows and cols that are multiples of 16, got {rows} x {cols}")
    return out.reshape(rows, cols) if inverse else out


def gemm_bf16(x: np.ndarray, w: np.ndarray, magnitude: bool = False):
    """x W^T in double from BF16 bit patterns (x: m x k, w: n x k); with
    magnitude also the sums of |x_t w_t| (for rounding-error bounds)."""
    x = np.ascontiguousarray(x, np.uint16)
    w = np.ascontiguousarray(w, np.uint16)
    m, k = x.shape
    n, k2 = w.shape
    if k != k2:
        raise ValueError("inner dimensions differ")
    y = np.zeros((m, n), np.float64)
    mag = np.zeros((m, n), np.float64)
    if y.size and k:
        lib().wco_gemm_bf16(_p(x), _p(w), m, n, k, _p(y), _p(mag))
    return (y, mag) if magnitude else y


# ------------------------------------------------------------ whole tensor

@dataclass
class Encoded:
    dtype: str
    n: int
    raw: np.ndarray      # uint8
    tables: np.ndarray   # uint16, chunks x 256 (1 x 256 with a tensor table)
    seek: np.ndarray     # uint64, chunks + 1
    payload: np.ndarray  # uint8, seek[-1] bytes
    opts: int = 0        # option bits

    @property
    def total_bytes(self) -> int:
        return int(self.raw.size + self.tables.nbytes + self.seek.nbytes + self.payload.size)


def encode(x: np.ndarray, dtype: str = "bf16", threads: int = 1, opts: int = 0) -> Encoded:
    """Encode the flat bit patterns of x (uint32 for fp32, uint16 otherwise)."""
    x = np.ascontiguousarray(x).view(elem_type(dtype)).ravel()
    lay = query_layout(dtype, x.size, opts)
    raw = np.zeros(lay.raw_bytes, np.uint8)
    tables = np.zeros(lay.table_bytes // 2, np.uint16)
    seek = np.zeros(lay.num_chunks + 1, np.uint64)
    payload = np.zeros(max(lay.payload_capacity, 1), np.uint8)
    rc = lib().wco_encode(_dt(dtype, opts), _p(x), x.size, _p(raw), _p(tables), _p(seek),
                          _p(payload), lay.payload_capacity, threads)
    if rc != OK:
        raise RuntimeError(f"wco_encode failed: {rc}")
    return Encoded(dtype, x.size, raw, tables.reshape(-1, 256), seek,
                   payload[: int(seek[-1])].copy(), opts)


def decode(e: Encoded, threads: int = 1, strict: bool = True):
    """Decode to the flat bit patterns; returns (array, error_bits)."""
    out = np.zeros(e.n, elem_type(e.dtype))
    err = ctypes.c_uint32(0)
    payload = np.ascontiguousarray(e.payload, np.uint8)
    pay = payload if payload.size else np.zeros(1, np.uint8)
    tables = np.ascontiguousarray(e.tables, np.uint16)
    tables = tables if tables.size else np.zeros(256, np.uint16)
    rc = lib().wco_decode(_dt(e.dtype, e.opts), _p(np.ascontiguousarray(e.raw, np.uint8)),
                          _p(tables),
                          _p(np.ascontiguousarray(e.seek, np.uint64)), _p(pay), payload.size, e.n,
                          _p(out), threads, ctypes.byref(err))
    if rc not in (OK, ERR_CORRUPT):
        raise RuntimeError(f"wco_decode failed: {rc}")
    if strict and rc != OK:
        raise ValueError(f"corrupt stream, error bits {err.value:#x}")
    return out, int(err.value)


# ------------------------------------------------------------------ batch

def plan_batch(dtype, ns, opts: int = 0):
    ns = np.ascontiguousarray(ns, np.uint64)
    cb = np.zeros(max(ns.size, 1), np.uint64)
    rb = np.zeros(max(ns.size, 1), np.uint64)
    tot = _Layout()
    lib().wco_plan_batch(_dt(dtype, opts), _p(ns), ns.size, _p(cb), _p(rb), ctypes.byref(tot))
    return cb[: ns.size], rb[: ns.size], Layout(tot.n, tot.num_chunks, tot.raw_bytes,
                                                  tot.table_bytes, tot.seek_bytes,
                                                  tot.payload_capacity)


@dataclass
class EncodedBatch:
    dtype: str
    ns: list
    raw: np.ndarray
    tables: np.ndarray
    seek: np.ndarray
    payload: np.ndarray
    opts: int = 0


def encode_batch(xs, dtype: str = "bf16", threads: int = 1, opts: int = 0) -> EncodedBatch:
    arrs = [np.ascontiguousarray(x).view(elem_type(dtype)).ravel() for x in xs]
    ns = np.array([a.size for a in arrs], np.uint64)
    _, _, tot = plan_batch(dtype, ns, opts)
    raw = np.zeros(max(tot.raw_bytes, 1), np.uint8)
    tables = np.zeros(max(tot.table_bytes // 2, 1), np.uint16)
    seek = np.zeros(tot.num_chunks + 1, np.uint64)
    payload = np.zeros(max(tot.payload_capacity, 1), np.uint8)
    ptrs = (ctypes.c_void_p * max(len(arrs), 1))(*[a.ctypes.data for a in arrs])
    rc = lib().wco_encode_batch(_dt(dtype, opts), ptrs, _p(ns), len(arrs), _p(raw), _p(tables),
                                _p(seek), _p(payload), tot.payload_capacity, threads)
    if rc != OK:
        raise RuntimeError(f"wco_encode_batch failed: {rc}")
    return EncodedBatch(dtype, [int(v) for v in ns], raw[: tot.raw_bytes],
                        tables[: tot.table_bytes // 2].reshape(-1, 256), seek,
                        payload[: int(seek[-1])].copy(), opts)


def decode_batch(e: EncodedBatch, threads: int = 1):
    outs = [np.zeros(n, elem_type(e.dtype)) for n in e.ns]
    ns = np.array(e.ns, np.uint64)
    ptrs = (ctypes.c_void_p * max(len(outs), 1))(*[o.ctypes.data for o in outs])
    err = ctypes.c_uint32(0)
    raw = e.raw if e.raw.size else np.zeros(1, np.uint8)
    tables = np.ascontiguousarray(e.tables, np.uint16)
    tables = tables if tables.size else np.zeros(1, np.uint16)
    pay = e.payload if e.payload.size else np.zeros(1, np.uint8)
    rc = lib().wco_decode_batch(_dt(e.dtype, e.opts), ptrs, _p(ns), len(outs), _p(raw), _p(tables),
                                _p(np.ascontiguousarray(e.seek, np.uint64)), _p(pay),
                                e.payload.size, threads, ctypes.byref(err))
    if rc not in (OK, ERR_CORRUPT):
        raise RuntimeError(f"wco_decode_batch failed: {rc}")
    return outs, int(err.value)
