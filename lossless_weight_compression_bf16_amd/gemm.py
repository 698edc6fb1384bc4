"""Decode fused with its consumer: Y += X W^T straight from compressed weights.

The serving side of the Split12 README (weights kept compressed in GPU memory
and decompressed inside the kernels that use them) as one HIP kernel: every
decoded 16 x 16 tile of W goes from the rANS decoder's registers into the
matrix cores (MFMA 16x16x16 bf16); no decoded copy of W is written.

Weights are encoded in tile order (``to_tiles``: 16 x 16 tiles, panel by
panel, each in the operand order of the matrix cores), which is a
permutation: ``decode_weights`` gives the row-major tensors back bit for bit.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _binding as B
from . import codec


def _check_w(w: torch.Tensor):
    codec._check_device(w)
    if w.dim() != 2 or w.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError("a weight must be a 2-D bfloat16 tensor (rows x cols)")
    if w.shape[0] % 16 or w.shape[1] % 16:
        raise ValueError(f"rows and cols must be multiples of 16, got {tuple(w.shape)}")


def to_tiles(w: torch.Tensor, stream=None) -> torch.Tensor:
    """The tile-ordered copy of a rows x cols BF16 matrix (flat)."""
    _check_w(w)
    src = w.contiguous()
    out = torch.empty(w.numel(), dtype=w.dtype, device=w.device)
    B.wc_tile_order(src, out, w.shape[0], w.shape[1], False, stream)
    return out


def from_tiles(t: torch.Tensor, rows: int, cols: int, stream=None) -> torch.Tensor:
    """The rows x cols matrix back from its tile-ordered values."""
    codec._check_device(t)
    if t.numel() != rows * cols:
        raise ValueError("size does not match the shape")
    out = torch.empty((rows, cols), dtype=t.dtype, device=t.device)
    B.wc_tile_order(t.contiguous(), out, rows, cols, True, stream)
    return out


@dataclass
class EncodedWeights:
    """BF16 weight matrices encoded in tile order (one batch)."""
    batch: codec.EncodedBatch
    shapes: list  # (rows, cols) per matrix

    @property
    def ratio(self) -> float:
        return self.batch.ratio


def encode_weights(ws, stream=None, reorder: bool = False, tensor_table: bool = False,
                   crc: bool = False) -> EncodedWeights:
    """Encode rows x cols BF16 matrices for the fused decode + GEMM."""
    if not ws:
        raise ValueError("empty batch")
    for w in ws:
        _check_w(w)
    tiles = [to_tiles(w, stream) for w in ws]
    e = codec.encode_batch(tiles, stream, reorder=reorder, tensor_table=tensor_table, crc=crc)
    return EncodedWeights(e, [(int(w.shape[0]), int(w.shape[1])) for w in ws])


def decode_weights(e: EncodedWeights, stream=None):
    """The row-major matrices, bit for bit."""
    tiles = codec.decode_batch(e.batch, stream=stream)
    return [from_tiles(t, r, c, stream) for t, (r, c) in zip(tiles, e.shapes)]


def gemm_descriptors(xs, ys, shapes):
    """Host array of wc_gemm descriptors for (X_i, Y_i, W_i shape)."""
    arr = (B.wc_gemm * len(shapes))()
    for i, ((r, c), x, y) in enumerate(zip(shapes, xs, ys)):
        arr[i].x, arr[i].y, arr[i].rows, arr[i].cols = x.data_ptr(), y.data_ptr(), r, c
    return arr


def descriptors_to_device(arr, dev) -> torch.Tensor:
    nbytes = ctypes.sizeof(arr)
    host = torch.frombuffer(bytearray(ctypes.string_at(ctypes.addressof(arr), nbytes)), dtype=torch.uint8)
    return host.to(dev)


def decode_gemm(e: EncodedWeights, xs, ys=None, stream=None, check: bool = True):
    """Y_i += X_i W_i^T for every matrix of the batch (X_i: m x cols_i BF16;
    Y_i: m x rows_i fp32, zeros when not given); returns the Y_i."""
    if len(xs) != len(e.shapes):
        raise ValueError("one X per matrix")
    dev = e.batch.seek.device
    m = int(xs[0].shape[0])
    for x, (r, c) in zip(xs, e.shapes):
        codec._check_device(x)
        if x.dtype != torch.bfloat16 or tuple(x.shape) != (m, c) or not x.is_contiguous():
            raise ValueError(f"X must be a contiguous {m} x {c} bfloat16 tensor")
    if ys is None:
        ys = [torch.zeros((m, r), dtype=torch.float32, device=dev) for r, _ in e.shapes]
    for y, (r, _) in zip(ys, e.shapes):
        if y.dtype != torch.float32 or tuple(y.shape) != (m, r) or not y.is_contiguous():
            raise ValueError(f"Y must be a contiguous {m} x {r} float32 tensor")
    ns = [r * c for r, c in e.shapes]
    h_segs, tot = B.wc_plan_batch(e.batch.fmt or e.batch.dtype, ns)
    d_segs = codec.segments_to_device(h_segs, len(ns), dev)
    h_g = gemm_descriptors(xs, ys, e.shapes)
    d_g = descriptors_to_device(h_g, dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    B.wc_decode_gemm_batch(e.batch.fmt or e.batch.dtype, h_segs, d_segs, len(ns), h_g, d_g, m, e.batch.buffers(),
                           err, stream)
    if check:
        codec._raise_bits(int(err.item()), "decode_gemm")
    return ys
