"""Tensor-level API over the C ABI: lossless encode / decode of BF16, FP16 and
FP32 weights (and FP8) on the GPU.

BF16 is split into its high byte (sign + 7 exponent bits), which is rANS
coded per 65536-element chunk, and its low byte, which is stored raw (the
weight-compression / Split12 README's byte split); FP32 keeps sign bits and
three mantissa bytes raw and codes the exponent byte (the SMEF README's
sign / exponent / mantissa streams); FP16 takes the same 2-plane byte split
as BF16; FP8 (E4M3, E5M2) is split into the exponent nibble, which is coded,
and the other nibble, stored raw two per byte.  Options: ``reorder`` applies the PTWM README's bit reorder first
(16-bit layouts: the coded byte starts with the whole exponent), and
``tensor_table`` / ``raw_fallback`` select one table per tensor and raw
storage of chunks that do not shrink; ``crc`` adds a CRC-32 per chunk that
decode checks on the GPU.  Tensors are handled as bit patterns
(uint16 / int32 views), never converted, so every pattern round-trips.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import _binding as B


def _dtype_of(t: torch.Tensor, reorder: bool = False) -> str:
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return "bf16r" if reorder else "bf16"
    if t.dtype == torch.float16:
        return "fp16r" if reorder else "fp16"
    if t.dtype in (torch.float32, torch.int32, torch.uint32):
        return "fp32"
    if t.dtype == torch.float8_e4m3fn:
        return "fp8e4m3"
    if t.dtype == torch.float8_e5m2:
        return "fp8e5m2"
    raise TypeError(f"unsupported dtype {t.dtype}: expected bfloat16, float16, float32 or float8")


def _bits(t: torch.Tensor, dtype) -> torch.Tensor:
    t = t.contiguous().reshape(-1)
    t = t.view({4: torch.int32, 2: torch.int16, 1: torch.uint8}[B.elem_bytes(dtype)])
    if t.numel() and t.data_ptr() % 16:
        t = t.clone()
    return t


def _check_device(t: torch.Tensor):
    if not t.is_cuda:
        raise ValueError("the codec runs on the GPU: move the tensor to a HIP device first")


@dataclass
class Encoded:
    """One encoded tensor; every buffer is a device tensor."""
    dtype: str                 # layout: "bf16", "bf16r", "fp16", "fp16r" or "fp32"
    n: int                     # elements
    shape: tuple
    torch_dtype: torch.dtype
    raw: torch.Tensor          # uint8, raw planes
    tables: torch.Tensor       # int16 (u16 bit patterns), chunks x 256
    seek: torch.Tensor         # int64 (u64), chunks + 1
    payload: torch.Tensor      # uint8, seek[-1] bytes
    fmt: int = 0               # format word (layout | options)
    crc: torch.Tensor | None = None  # int32 (u32 CRC-32 per chunk), with the CRC option

    @property
    def num_chunks(self) -> int:
        return int(self.seek.numel() - 1)

    @property
    def compressed_bytes(self) -> int:
        return int(self.raw.numel() + self.tables.numel() * 2 + self.seek.numel() * 8 + self.payload.numel()
                   + (self.crc.numel() * 4 if self.crc is not None else 0))

    @property
    def raw_input_bytes(self) -> int:
        return self.n * B.elem_bytes(self.dtype)

    @property
    def ratio(self) -> float:
        return self.compressed_bytes / max(self.raw_input_bytes, 1)

    def buffers(self) -> B.wc_buffers:
        return B.make_buffers(self.raw, self.tables, self.seek, self.payload, self.payload.numel(), self.crc)

    def to_host(self) -> dict:
        h = {"raw": self.raw.cpu().numpy(), "tables": self.tables.cpu().numpy().view("<u2"),
             "seek": self.seek.cpu().numpy().view("<u8"), "payload": self.payload.cpu().numpy()}
        if self.crc is not None:
            h["crc"] = self.crc.cpu().numpy().view("<u4")
        return h


def _raise_bits(bits: int, what: str):
    if bits:
        raise B.WcError(f"{what}: device reported {', '.join(B.error_names(bits))} (bits {bits:#x})")


def _layout_for(t: torch.Tensor, layout, reorder: bool) -> str:
    """The plane layout: named explicitly (for tensors of raw bit patterns,
    e.g. uint8 holding FP8), or from the tensor's float type."""
    if layout is None:
        return _dtype_of(t, reorder)
    if layout not in B.DTYPE_CODES:
        raise ValueError(f"unknown layout {layout!r}")
    if t.element_size() != B.elem_bytes(layout):
        raise TypeError(f"layout {layout} takes {B.elem_bytes(layout)}-byte elements, not {t.dtype}")
    return layout


def encode(t: torch.Tensor, stream=None, reorder: bool = False, tensor_table: bool = False,
           raw_fallback: bool = False, layout: str | None = None, crc: bool = False) -> Encoded:
    """Losslessly encode a bf16 / fp16 / fp32 / fp8 device tensor (synchronises
    once to size the payload)."""
    _check_device(t)
    dtype = _layout_for(t, layout, reorder)
    fmt = B.format_word(dtype, tensor_table, raw_fallback, crc)
    x = _bits(t, dtype)
    n = x.numel()
    dev = x.device
    lay = B.wc_query_layout(fmt, n)
    raw = torch.empty(max(lay.raw_bytes, 1), dtype=torch.uint8, device=dev)
    tables = torch.empty(max(lay.table_bytes // 2, 8), dtype=torch.int16, device=dev)
    seek = torch.empty(lay.num_chunks + 1, dtype=torch.int64, device=dev)
    payload = torch.empty(max(lay.payload_capacity, 16), dtype=torch.uint8, device=dev)
    scratch = torch.empty(max(lay.scratch_bytes, 256), dtype=torch.uint8, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    crcs = torch.empty(max(lay.num_chunks, 1), dtype=torch.int32, device=dev) if crc else None
    bufs = B.make_buffers(raw, tables, seek, payload, lay.payload_capacity, crcs)
    B.wc_encode(fmt, x, n, bufs, scratch, scratch.numel(), err, stream)
    total = int(seek[-1].item())
    _raise_bits(int(err.item()), "encode")
    del scratch
    return Encoded(dtype, n, tuple(t.shape), t.dtype, raw[: lay.raw_bytes],
                   tables[: lay.table_bytes // 2].view(-1, 256), seek, payload[:total].clone(), fmt,
                   crcs[: lay.num_chunks] if crc else None)


def decode(e: Encoded, out: torch.Tensor | None = None, stream=None, check: bool = True) -> torch.Tensor:
    """Decode to a tensor of the original shape and dtype (bit-identical)."""
    dev = e.seek.device
    if out is None:
        out = torch.empty(e.shape, dtype=e.torch_dtype, device=dev)
    x = _bits(out, e.dtype) if out.is_contiguous() else None
    if x is None or x.data_ptr() != out.data_ptr():
        raise ValueError("out must be a contiguous, 16-byte aligned tensor")
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    B.wc_decode(e.fmt or e.dtype, e.buffers(), e.n, x, err, stream)
    if check:
        _raise_bits(int(err.item()), "decode")
    return out


@dataclass
class EncodedBatch:
    """A set of tensors coded in one launch sequence; chunks of tensor i
    follow those of tensor i-1 in tables / seek / payload."""
    dtype: str
    ns: list
    shapes: list
    torch_dtype: torch.dtype
    raw: torch.Tensor
    tables: torch.Tensor
    seek: torch.Tensor
    payload: torch.Tensor
    h_segs: object = field(repr=False, default=None)
    fmt: int = 0
    crc: torch.Tensor | None = None

    @property
    def compressed_bytes(self) -> int:
        return int(self.raw.numel() + self.tables.numel() * 2 + self.seek.numel() * 8 + self.payload.numel()
                   + (self.crc.numel() * 4 if self.crc is not None else 0))

    @property
    def raw_input_bytes(self) -> int:
        return sum(self.ns) * B.elem_bytes(self.dtype)

    @property
    def ratio(self) -> float:
        return self.compressed_bytes / max(self.raw_input_bytes, 1)

    def buffers(self) -> B.wc_buffers:
        return B.make_buffers(self.raw, self.tables, self.seek, self.payload, self.payload.numel(), self.crc)


def _segments(dtype, xs, dev):
    h_segs, tot = B.wc_plan_batch(dtype, [x.numel() for x in xs])
    for i, x in enumerate(xs):
        h_segs[i].ptr = x.data_ptr() if x.numel() else 0
    d_segs = segments_to_device(h_segs, len(xs), dev)
    return h_segs, d_segs, tot


def segments_to_device(h_segs, nseg: int, dev) -> torch.Tensor:
    import ctypes
    nbytes = ctypes.sizeof(B.wc_segment) * nseg
    host = torch.frombuffer(bytearray(ctypes.string_at(ctypes.addressof(h_segs), nbytes)),
                            dtype=torch.uint8)
    return host.to(dev)


def encode_batch(ts, stream=None, reorder: bool = False, tensor_table: bool = False,
                 raw_fallback: bool = False, layout: str | None = None, crc: bool = False) -> EncodedBatch:
    """Encode a list of same-dtype device tensors in one launch sequence."""
    if not ts:
        raise ValueError("empty batch")
    for t in ts:
        _check_device(t)
    dtype = _layout_for(ts[0], layout, reorder)
    if any(_layout_for(t, layout, reorder) != dtype for t in ts):
        raise TypeError("all tensors of a batch must share a dtype")
    fmt = B.format_word(dtype, tensor_table, raw_fallback, crc)
    xs = [_bits(t, dtype) for t in ts]
    dev = xs[0].device
    h_segs, d_segs, tot = _segments(fmt, xs, dev)
    raw = torch.empty(max(tot.raw_bytes, 16), dtype=torch.uint8, device=dev)
    tables = torch.empty(max(tot.table_bytes // 2, 8), dtype=torch.int16, device=dev)
    seek = torch.empty(tot.num_chunks + 1, dtype=torch.int64, device=dev)
    payload = torch.empty(max(tot.payload_capacity, 16), dtype=torch.uint8, device=dev)
    scratch = torch.empty(max(tot.scratch_bytes, 256), dtype=torch.uint8, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    crcs = torch.empty(max(tot.num_chunks, 1), dtype=torch.int32, device=dev) if crc else None
    bufs = B.make_buffers(raw, tables, seek, payload, tot.payload_capacity, crcs)
    B.wc_encode_batch(fmt, h_segs, d_segs, len(xs), bufs, scratch, scratch.numel(), err, stream)
    total = int(seek[-1].item())
    _raise_bits(int(err.item()), "encode_batch")
    del scratch
    return EncodedBatch(dtype, [x.numel() for x in xs], [tuple(t.shape) for t in ts], ts[0].dtype,
                        raw[: tot.raw_bytes], tables[: tot.table_bytes // 2].view(-1, 256), seek,
                        payload[:total].clone(), h_segs, fmt, crcs[: tot.num_chunks] if crc else None)


def decode_batch(e: EncodedBatch, outs=None, stream=None, check: bool = True):
    """Decode every tensor of a batch in one launch."""
    dev = e.seek.device
    if outs is None:
        outs = [torch.empty(s, dtype=e.torch_dtype, device=dev) for s in e.shapes]
    xs = [_bits(o, e.dtype) for o in outs]
    for o, x in zip(outs, xs):
        if x.numel() and x.data_ptr() != o.data_ptr():
            raise ValueError("outputs must be contiguous and 16-byte aligned")
    fmt = e.fmt or e.dtype
    h_segs, d_segs, _ = _segments(fmt, xs, dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    B.wc_decode_batch(fmt, h_segs, d_segs, len(xs), e.buffers(), err, stream)
    if check:
        _raise_bits(int(err.item()), "decode_batch")
    return outs
