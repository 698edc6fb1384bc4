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

BF16 = 0
FP32 = 1
DTYPES = {"bf16": BF16, "fp32": FP32}

OK, ERR_ARG, ERR_CAPACITY, ERR_CORRUPT = 0, 1, 2, 3
EF_BAD_TABLE, EF_WORD_OVERRUN, EF_BAD_FINAL_STATE, EF_BAD_TAIL, EF_BAD_SEEK = 1, 2, 4, 8, 16

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


def _dt(dtype) -> int:
    return DTYPES[dtype] if isinstance(dtype, str) else int(dtype)


@dataclass
class Layout:
    n: int
    num_chunks: int
    raw_bytes: int
    table_bytes: int
    seek_bytes: int
    payload_capacity: int


def query_layout(dtype, n: int) -> Layout:
    out = _Layout()
    rc = lib().wco_query_layout(_dt(dtype), n, ctypes.byref(out))
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


# ------------------------------------------------------------ whole tensor

@dataclass
class Encoded:
    dtype: str
    n: int
    raw: np.ndarray      # uint8
    tables: np.ndarray   # uint16, chunks x 256
    seek: np.ndarray     # uint64, chunks + 1
    payload: np.ndarray  # uint8, seek[-1] bytes

    @property
    def total_bytes(self) -> int:
        return int(self.raw.size + self.tables.nbytes + self.seek.nbytes + self.payload.size)


def encode(x: np.ndarray, dtype: str = "bf16", threads: int = 1) -> Encoded:
    """Encode the flat bit patterns of x (uint16 for bf16, uint32 for fp32)."""
    want = np.uint16 if dtype == "bf16" else np.uint32
    x = np.ascontiguousarray(x).view(want).ravel()
    lay = query_layout(dtype, x.size)
    raw = np.zeros(lay.raw_bytes, np.uint8)
    tables = np.zeros(lay.num_chunks * 256, np.uint16)
    seek = np.zeros(lay.num_chunks + 1, np.uint64)
    payload = np.zeros(max(lay.payload_capacity, 1), np.uint8)
    rc = lib().wco_encode(_dt(dtype), _p(x), x.size, _p(raw), _p(tables), _p(seek), _p(payload),
                          lay.payload_capacity, threads)
    if rc != OK:
        raise RuntimeError(f"wco_encode failed: {rc}")
    return Encoded(dtype, x.size, raw, tables.reshape(-1, 256), seek,
                   payload[: int(seek[-1])].copy())


def decode(e: Encoded, threads: int = 1, strict: bool = True):
    """Decode to the flat bit patterns; returns (array, error_bits)."""
    want = np.uint16 if e.dtype == "bf16" else np.uint32
    out = np.zeros(e.n, want)
    err = ctypes.c_uint32(0)
    payload = np.ascontiguousarray(e.payload, np.uint8)
    pay = payload if payload.size else np.zeros(1, np.uint8)
    rc = lib().wco_decode(_dt(e.dtype), _p(np.ascontiguousarray(e.raw, np.uint8)),
                          _p(np.ascontiguousarray(e.tables, np.uint16)),
                          _p(np.ascontiguousarray(e.seek, np.uint64)), _p(pay), payload.size, e.n,
                          _p(out), threads, ctypes.byref(err))
    if rc not in (OK, ERR_CORRUPT):
        raise RuntimeError(f"wco_decode failed: {rc}")
    if strict and rc != OK:
        raise ValueError(f"corrupt stream, error bits {err.value:#x}")
    return out, int(err.value)


# ------------------------------------------------------------------ batch

def plan_batch(dtype, ns):
    ns = np.ascontiguousarray(ns, np.uint64)
    cb = np.zeros(max(ns.size, 1), np.uint64)
    rb = np.zeros(max(ns.size, 1), np.uint64)
    tot = _Layout()
    lib().wco_plan_batch(_dt(dtype), _p(ns), ns.size, _p(cb), _p(rb), ctypes.byref(tot))
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


def encode_batch(xs, dtype: str = "bf16", threads: int = 1) -> EncodedBatch:
    want = np.uint16 if dtype == "bf16" else np.uint32
    arrs = [np.ascontiguousarray(x).view(want).ravel() for x in xs]
    ns = np.array([a.size for a in arrs], np.uint64)
    _, _, tot = plan_batch(dtype, ns)
    raw = np.zeros(max(tot.raw_bytes, 1), np.uint8)
    tables = np.zeros(max(tot.num_chunks * 256, 1), np.uint16)
    seek = np.zeros(tot.num_chunks + 1, np.uint64)
    payload = np.zeros(max(tot.payload_capacity, 1), np.uint8)
    ptrs = (ctypes.c_void_p * max(len(arrs), 1))(*[a.ctypes.data for a in arrs])
    rc = lib().wco_encode_batch(_dt(dtype), ptrs, _p(ns), len(arrs), _p(raw), _p(tables),
                                _p(seek), _p(payload), tot.payload_capacity, threads)
    if rc != OK:
        raise RuntimeError(f"wco_encode_batch failed: {rc}")
    return EncodedBatch(dtype, [int(v) for v in ns], raw[: tot.raw_bytes],
                        tables[: tot.num_chunks * 256].reshape(-1, 256), seek,
                        payload[: int(seek[-1])].copy())


def decode_batch(e: EncodedBatch, threads: int = 1):
    want = np.uint16 if e.dtype == "bf16" else np.uint32
    outs = [np.zeros(n, want) for n in e.ns]
    ns = np.array(e.ns, np.uint64)
    ptrs = (ctypes.c_void_p * max(len(outs), 1))(*[o.ctypes.data for o in outs])
    err = ctypes.c_uint32(0)
    raw = e.raw if e.raw.size else np.zeros(1, np.uint8)
    tables = np.ascontiguousarray(e.tables, np.uint16)
    tables = tables if tables.size else np.zeros(1, np.uint16)
    pay = e.payload if e.payload.size else np.zeros(1, np.uint8)
    rc = lib().wco_decode_batch(_dt(e.dtype), ptrs, _p(ns), len(outs), _p(raw), _p(tables),
                                _p(np.ascontiguousarray(e.seek, np.uint64)), _p(pay),
                                e.payload.size, threads, ctypes.byref(err))
    if rc not in (OK, ERR_CORRUPT):
        raise RuntimeError(f"wco_decode_batch failed: {rc}")
    return outs, int(err.value)
