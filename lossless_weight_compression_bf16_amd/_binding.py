"""ctypes binding of libwc.so (the C ABI in include/wc.h).

Argument marshalling only: every step of the codec runs in the HIP kernels
behind the C ABI; torch provides device memory and the current HIP stream.
The library is loaded on first use and a missing build is an error, never a
fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwc.so")

WC_BF16, WC_FP32, WC_BF16_REORDER, WC_FP16, WC_FP16_REORDER, WC_FP8_E4M3, WC_FP8_E5M2 = 0, 1, 2, 3, 4, 5, 6
DTYPE_CODES = {"bf16": WC_BF16, "fp32": WC_FP32, "bf16r": WC_BF16_REORDER, "fp16": WC_FP16,
               "fp16r": WC_FP16_REORDER, "fp8e4m3": WC_FP8_E4M3, "fp8e5m2": WC_FP8_E5M2}
WC_OPT_TENSOR_TABLE = 0x100
WC_OPT_RAW_FALLBACK = 0x200
WC_OPT_CRC32 = 0x400

WC_OK, WC_ERR_ARG, WC_ERR_CAPACITY, WC_ERR_CORRUPT, WC_ERR_HIP = 0, 1, 2, 3, 4
EF_BAD_TABLE = 1
EF_WORD_OVERRUN = 2
EF_BAD_FINAL_STATE = 4
EF_BAD_TAIL = 8
EF_BAD_SEEK = 16
EF_CAPACITY = 32
EF_BAD_CRC = 64
EF_NAMES = {EF_BAD_TABLE: "bad table", EF_WORD_OVERRUN: "word overrun",
            EF_BAD_FINAL_STATE: "bad final state", EF_BAD_TAIL: "bad tail",
            EF_BAD_SEEK: "bad seek", EF_CAPACITY: "payload capacity", EF_BAD_CRC: "CRC mismatch"}

CHUNK = 65536
WC_NOALLOC_SCRATCH_BYTES = 128 << 20  # the fixed device array of wc_encode_noalloc

EXPORTS = ["wc_version", "wc_status_string", "wc_query_layout", "wc_plan_batch", "wc_encode",
           "wc_decode", "wc_encode_batch", "wc_decode_batch", "wc_check_division", "wc_tile_order",
           "wc_decode_gemm_batch", "wc_decode_variant", "wc_encode_noalloc", "wc_noalloc_max_chunks",
           "wc_set_encoder_words", "wc_encode_variant"]
# encoder word-store forms (wc_set_encoder_words)
ENC_WORDS_AUTO, ENC_WORDS_DIRECT, ENC_WORDS_STAGED = 0, 1, 2


class WcError(RuntimeError):
    """A non-OK status from the C ABI, or error bits reported by a kernel."""


class wc_layout(ctypes.Structure):
    _fields_ = [("n", ctypes.c_uint64), ("num_chunks", ctypes.c_uint64),
                ("raw_bytes", ctypes.c_uint64), ("table_bytes", ctypes.c_uint64),
                ("seek_bytes", ctypes.c_uint64), ("payload_capacity", ctypes.c_uint64),
                ("scratch_bytes", ctypes.c_uint64), ("crc_bytes", ctypes.c_uint64)]

    def as_dict(self):
        return {k: int(getattr(self, k)) for k, _ in self._fields_}


class wc_buffers(ctypes.Structure):
    _fields_ = [("raw", ctypes.c_void_p), ("tables", ctypes.c_void_p), ("seek", ctypes.c_void_p),
                ("payload", ctypes.c_void_p), ("payload_bytes", ctypes.c_uint64), ("crc", ctypes.c_void_p)]


class wc_segment(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_uint64), ("n", ctypes.c_uint64), ("chunk_base", ctypes.c_uint64),
                ("raw_base", ctypes.c_uint64)]


class wc_gemm(ctypes.Structure):
    _fields_ = [("x", ctypes.c_uint64), ("y", ctypes.c_uint64), ("rows", ctypes.c_uint32),
                ("cols", ctypes.c_uint32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libwc.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise WcError(f"{LIB_PATH} is missing: build the HIP library first "
                      "(python -m lossless_weight_compression_bf16_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    P, U64, U32, I = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int
    L.wc_version.restype = I
    L.wc_status_string.argtypes = [I]
    L.wc_status_string.restype = ctypes.c_char_p
    L.wc_query_layout.argtypes = [I, U64, ctypes.POINTER(wc_layout)]
    L.wc_plan_batch.argtypes = [I, P, U32, ctypes.POINTER(wc_layout)]
    L.wc_encode.argtypes = [I, P, U64, ctypes.POINTER(wc_buffers), P, U64, P, P, P]
    L.wc_decode.argtypes = [I, ctypes.POINTER(wc_buffers), U64, P, P, P]
    L.wc_encode_batch.argtypes = [I, P, P, U32, ctypes.POINTER(wc_buffers), P, U64, P, P, P]
    L.wc_decode_batch.argtypes = [I, P, P, U32, ctypes.POINTER(wc_buffers), P, P]
    L.wc_check_division.argtypes = [U32]
    L.wc_check_division.restype = U64
    L.wc_tile_order.argtypes = [P, P, U32, U32, I, P]
    L.wc_decode_gemm_batch.argtypes = [I, P, P, U32, P, P, U32, ctypes.POINTER(wc_buffers), P, P]
    L.wc_decode_variant.argtypes = [I, U64, U64, U64, P, ctypes.POINTER(I), ctypes.POINTER(I)]
    L.wc_encode_noalloc.argtypes = [I, P, U64, ctypes.POINTER(wc_buffers), P, P]
    L.wc_set_encoder_words.argtypes = [I]
    L.wc_set_encoder_words.restype = I
    L.wc_encode_variant.argtypes = [I, U64, P, ctypes.POINTER(I)]
    L.wc_noalloc_max_chunks.argtypes = [I]
    L.wc_noalloc_max_chunks.restype = U64
    for name in ("wc_query_layout", "wc_plan_batch", "wc_encode", "wc_decode", "wc_encode_batch",
                 "wc_decode_batch", "wc_tile_order", "wc_decode_gemm_batch", "wc_decode_variant",
                 "wc_encode_noalloc", "wc_encode_variant"):
        getattr(L, name).restype = I
    _lib = L
    return L


def _check(rc: int, what: str):
    if rc != WC_OK:
        msg = lib().wc_status_string(rc).decode()
        raise WcError(f"{what}: {msg} (status {rc})")


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return int(t.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _code(dtype) -> int:
    """Format word of a layout name, or an int format word as given."""
    return DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)


def format_word(dtype, tensor_table: bool = False, raw_fallback: bool = False, crc: bool = False) -> int:
    """A plane layout (name or code) OR-ed with the option bits."""
    return (_code(dtype) | (WC_OPT_TENSOR_TABLE if tensor_table else 0)
            | (WC_OPT_RAW_FALLBACK if raw_fallback else 0) | (WC_OPT_CRC32 if crc else 0))


def elem_bytes(fmt) -> int:
    layout = _code(fmt) & 0xFF
    return 4 if layout == WC_FP32 else 1 if layout in (WC_FP8_E4M3, WC_FP8_E5M2) else 2


def error_names(bits: int):
    return [name for bit, name in EF_NAMES.items() if bits & bit]


# ------------------------------------------------------------ C-ABI mirror

def wc_version() -> int:
    return int(lib().wc_version())


def wc_query_layout(dtype, n: int) -> wc_layout:
    out = wc_layout()
    _check(lib().wc_query_layout(_code(dtype), int(n), ctypes.byref(out)), "wc_query_layout")
    return out


def wc_plan_batch(dtype, ns):
    """Returns (segment array (ctypes), total layout) for element counts ns;
    the segment pointers are left 0 for the caller to fill."""
    segs = (wc_segment * max(len(ns), 1))()
    for i, n in enumerate(ns):
        segs[i].n = int(n)
    tot = wc_layout()
    _check(lib().wc_plan_batch(_code(dtype), segs, len(ns), ctypes.byref(tot)), "wc_plan_batch")
    return segs, tot


def make_buffers(raw, tables, seek, payload, payload_bytes: int, crc=None) -> wc_buffers:
    return wc_buffers(_ptr(raw), _ptr(tables), _ptr(seek), _ptr(payload), int(payload_bytes), _ptr(crc))


def wc_encode(dtype, d_in, n: int, bufs: wc_buffers, d_scratch, scratch_bytes: int, d_err=None,
              stream=None, stage_events=None):
    ev = _events_arg(stage_events, 5)
    rc = lib().wc_encode(_code(dtype), _ptr(d_in), int(n), ctypes.byref(bufs), _ptr(d_scratch),
                         int(scratch_bytes), _ptr(d_err), _stream(stream), ev)
    _check(rc, "wc_encode")


def wc_decode(dtype, bufs: wc_buffers, n: int, d_out, d_err=None, stream=None):
    rc = lib().wc_decode(_code(dtype), ctypes.byref(bufs), int(n), _ptr(d_out), _ptr(d_err),
                         _stream(stream))
    _check(rc, "wc_decode")


def wc_encode_batch(dtype, h_segs, d_segs, nseg: int, bufs: wc_buffers, d_scratch, scratch_bytes: int,
                    d_err=None, stream=None, stage_events=None):
    ev = _events_arg(stage_events, 5)
    rc = lib().wc_encode_batch(_code(dtype), ctypes.cast(h_segs, ctypes.c_void_p), _ptr(d_segs),
                               int(nseg), ctypes.byref(bufs), _ptr(d_scratch), int(scratch_bytes),
                               _ptr(d_err), _stream(stream), ev)
    _check(rc, "wc_encode_batch")


def wc_encode_noalloc(dtype, d_in, n: int, bufs: wc_buffers, d_err=None, stream=None):
    """wc_encode with the library's fixed device scratch (no allocation)."""
    rc = lib().wc_encode_noalloc(_code(dtype), _ptr(d_in), int(n), ctypes.byref(bufs), _ptr(d_err),
                                 _stream(stream))
    _check(rc, "wc_encode_noalloc")


def wc_noalloc_max_chunks(dtype) -> int:
    return int(lib().wc_noalloc_max_chunks(_code(dtype)))


def wc_decode_batch(dtype, h_segs, d_segs, nseg: int, bufs: wc_buffers, d_err=None, stream=None):
    rc = lib().wc_decode_batch(_code(dtype), ctypes.cast(h_segs, ctypes.c_void_p), _ptr(d_segs),
                               int(nseg), ctypes.byref(bufs), _ptr(d_err), _stream(stream))
    _check(rc, "wc_decode_batch")


def wc_tile_order(d_in, d_out, rows: int, cols: int, inverse: bool = False, stream=None):
    rc = lib().wc_tile_order(_ptr(d_in), _ptr(d_out), int(rows), int(cols), 1 if inverse else 0, _stream(stream))
    _check(rc, "wc_tile_order")


def wc_decode_gemm_batch(dtype, h_segs, d_segs, nseg: int, h_gemm, d_gemm, m: int, bufs: wc_buffers, d_err=None,
                         stream=None):
    rc = lib().wc_decode_gemm_batch(_code(dtype), ctypes.cast(h_segs, ctypes.c_void_p), _ptr(d_segs), int(nseg),
                                    ctypes.cast(h_gemm, ctypes.c_void_p), _ptr(d_gemm), int(m), ctypes.byref(bufs),
                                    _ptr(d_err), _stream(stream))
    _check(rc, "wc_decode_gemm_batch")


def wc_decode_variant(dtype, num_chunks: int, n: int, payload_bytes: int, stream=None):
    """(one_chunk_per_wave, refill_dwords) of the decoder the library would
    launch on the device of `stream`."""
    a, b = ctypes.c_int(0), ctypes.c_int(0)
    rc = lib().wc_decode_variant(_code(dtype), int(num_chunks), int(n), int(payload_bytes), _stream(stream),
                                 ctypes.byref(a), ctypes.byref(b))
    _check(rc, "wc_decode_variant")
    return bool(a.value), int(b.value)


def wc_set_encoder_words(mode: int) -> int:
    """Sets the encoder word-store form (ENC_WORDS_*) for the process;
    returns the previous one."""
    prev = int(lib().wc_set_encoder_words(int(mode)))
    if prev < 0:
        raise WcError(f"wc_set_encoder_words: bad mode {mode}")
    return prev


def wc_encode_variant(dtype, num_chunks: int, stream=None) -> bool:
    """True if an encode of num_chunks chunks would stage its words in LDS
    on the device of `stream`."""
    a = ctypes.c_int(0)
    rc = lib().wc_encode_variant(_code(dtype), int(num_chunks), _stream(stream), ctypes.byref(a))
    _check(rc, "wc_encode_variant")
    return bool(a.value)


def wc_check_division(samples_per_divisor: int = 256) -> int:
    return int(lib().wc_check_division(int(samples_per_divisor)))


# ------------------------------------------------------ HIP events (timing)

_hip = None


def _hiprt():
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so")
        h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                          ctypes.c_void_p]
        _hip = h
    return _hip


class HipEvents:
    """n raw hipEvent_t handles (for stage timing inside the library)."""

    def __init__(self, n: int):
        h = _hiprt()
        self.handles = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if h.hipEventCreate(ctypes.byref(ev)) != 0:
                raise WcError("hipEventCreate failed")
            self.handles[i] = ev.value

    def record(self, i: int, stream=None):
        _hiprt().hipEventRecord(self.handles[i], _stream(stream))

    def elapsed_ms(self, i: int, j: int) -> float:
        h = _hiprt()
        h.hipEventSynchronize(self.handles[j])
        out = ctypes.c_float()
        if h.hipEventElapsedTime(ctypes.byref(out), self.handles[i], self.handles[j]) != 0:
            raise WcError("hipEventElapsedTime failed")
        return float(out.value)

    def close(self):
        h = _hiprt()
        for v in self.handles:
            if v:
                h.hipEventDestroy(v)
        self.handles = (ctypes.c_void_p * 0)()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _events_arg(ev, n):
    if ev is None:
        return None
    if len(ev.handles) < n:
        raise ValueError(f"need {n} events")
    return ctypes.cast(ev.handles, ctypes.c_void_p)
