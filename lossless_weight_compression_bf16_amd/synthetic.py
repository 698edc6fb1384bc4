"""Seeded synthetic weight sets (host side, numpy).

Shared by the tests and the benchmark.  It holds no codec arithmetic: it only
draws random values and rounds them to BF16 / FP32 bit patterns.

The pages measure on trained checkpoints (GPT-2 in the SMEF README, a 753B
model in the weight-compression README, a BF16 GGUF in the SeedPack README)
that are not available here; these sets stand in for them with the same
shapes and with value distributions typical of trained weights.

Recipe
------
* Tensor ``i`` of a set and its block ``j`` of ``GEN_BLOCK`` consecutive
  elements draw from ``numpy.random.Generator(PCG64(SeedSequence(seed,
  spawn_key=(i, j))))``, so any block can be regenerated on its own (sampled
  checks at full size) and blocks can be drawn in parallel.  Per-tensor
  parameters (a random sigma) come from ``spawn_key=(i,)``.
* Normal values: float64 standard normals times sigma, rounded to float32.
  Outliers: after the normals, one uniform draw per element; with
  probability ``p_outlier`` the element becomes sign(draw) * k * sigma.
  Student-t: float64 t(nu) draws times scale.
* BF16: round-to-nearest-even of the float32 bit pattern,
  ``(u + 0x7FFF + ((u >> 16) & 1)) >> 16`` (what ``torch.to(bfloat16)`` does
  for finite values).
* FP16 (``with_dtype(w, "fp16")``): the same float32 values rounded to IEEE
  half by numpy (round to nearest even).
* FP8 (``with_dtype(w, "fp8e4m3")`` / ``"fp8e5m2"``): per tensor, the float32
  values scaled so the largest magnitude becomes the format's largest finite
  value (the usual per-tensor FP8 scaling), rounded by torch's float8 types.
  The scale depends on the whole tensor, so FP8 sets are generated a tensor
  at a time (``tensor_bits``), not block by block.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

GEN_BLOCK = 1 << 20
FP8_TYPES = {"fp8e4m3": "float8_e4m3fn", "fp8e5m2": "float8_e5m2"}


@dataclass(frozen=True)
class Dist:
    kind: str                   # "normal" or "student_t"
    sigma: float = 0.02         # normal: fixed std (when sigma_range is None)
    sigma_range: tuple | None = None  # normal: per-tensor sigma ~ U[lo, hi]
    p_outlier: float = 0.0      # normal: outlier probability per element
    outlier_k: float = 20.0     # outliers sit at +-k sigma
    nu: float = 3.0             # student_t degrees of freedom
    scale: float = 0.0          # student_t multiplier


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                  # "bf16", "fp16", "fp32", "fp8e4m3" or "fp8e5m2"
    shapes: tuple               # tuple of (rows, cols) in set order
    dist: Dist
    seed: int = 0
    note: str = ""

    @property
    def numels(self):
        return [int(r) * int(c) for r, c in self.shapes]

    @property
    def n(self) -> int:
        return sum(self.numels)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 1 if self.dtype in FP8_TYPES else 2

    @property
    def raw_bytes(self) -> int:
        return self.n * self.elem_bytes


def _gpt2_small():
    shapes = []
    for _ in range(12):
        shapes += [(768, 2304), (768, 768), (768, 3072), (3072, 768)]
    shapes.append((50257, 768))
    return tuple(shapes)


def _llama3_8b():
    shapes = []
    for _ in range(32):
        shapes += [(4096, 4096), (4096, 1024), (4096, 1024), (4096, 4096),
                   (4096, 14336), (4096, 14336), (14336, 4096)]
    shapes += [(128256, 4096), (128256, 4096)]
    return tuple(shapes)


def _moe_experts():
    shapes = []
    for _ in range(256):
        shapes += [(7168, 2048), (7168, 2048), (2048, 7168)]
    return tuple(shapes)


WORKLOADS = {
    w.name: w for w in [
        Workload("bf16-768x2304", "bf16", ((768, 2304),), Dist("normal", sigma=0.02),
                 note="one BF16 tensor, N(0, 0.02), seed 0"),
        Workload("gpt2-small-bf16", "bf16", _gpt2_small(),
                 Dist("normal", sigma_range=(0.01, 0.05)),
                 note="GPT-2-small-shaped BF16 set, 49 tensors, sigma_t ~ U[0.01, 0.05]"),
        Workload("fp32-768x2304", "fp32", ((768, 2304),), Dist("normal", sigma=0.02),
                 note="the float32 draws of bf16-768x2304 kept in FP32 (their BF16 rounding is that set)"),
        Workload("llama3-8b-bf16", "bf16", _llama3_8b(),
                 Dist("normal", sigma=0.02, p_outlier=1e-3, outlier_k=20.0),
                 note="Llama-3-8B-shaped BF16 set, 226 tensors, 0.1% outliers at 20 sigma"),
        Workload("moe-experts-bf16", "bf16", _moe_experts(),
                 Dist("student_t", nu=3.0, scale=0.015 / math.sqrt(3.0)),
                 note="256 experts x (w1, w3, w2), Student-t nu=3 scaled to std 0.015"),
        # the experts' down projections as weights of Y = X W^T (rows = 7168
        # output features, cols = 2048 inputs): the fused decode + GEMM set
        Workload("moe-w2-bf16", "bf16", tuple([(7168, 2048)] * 256),
                 Dist("student_t", nu=3.0, scale=0.015 / math.sqrt(3.0)), seed=5,
                 note="256 expert down projections, 7168 x 2048 (out x in), Student-t nu=3, std 0.015"),
    ]
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def with_dtype(w: Workload, dtype: str) -> Workload:
    """The same set (shapes, distribution, seed) stored as another float type."""
    if dtype == w.dtype:
        return w
    if w.dtype == "fp32" or dtype not in ("bf16", "fp16", *FP8_TYPES):
        raise ValueError(f"{w.name} cannot be stored as {dtype}")
    return Workload(f"{w.name}-as-{dtype}", dtype, w.shapes, w.dist, w.seed, w.note)


def _rng(seed: int, key: tuple) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def tensor_sigma(w: Workload, i: int) -> float:
    d = w.dist
    if d.kind != "normal":
        return float("nan")
    if d.sigma_range is None:
        return d.sigma
    lo, hi = d.sigma_range
    return float(_rng(w.seed, (i,)).uniform(lo, hi))


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16 bit patterns (finite inputs)."""
    u = x32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def block_f32(w: Workload, i: int, j: int) -> np.ndarray:
    """Float32 values of block j of tensor i."""
    n = w.numels[i]
    start = j * GEN_BLOCK
    length = min(GEN_BLOCK, n - start)
    if length <= 0:
        raise IndexError("block out of range")
    g = _rng(w.seed, (i, j))
    d = w.dist
    if d.kind == "normal":
        sigma = tensor_sigma(w, i)
        z = g.standard_normal(length)
        v = z * sigma
        if d.p_outlier > 0:
            u = g.random(length)
            m = u < d.p_outlier
            v[m] = np.sign(z[m]) * d.outlier_k * sigma
        return v.astype(np.float32)
    if d.kind == "student_t":
        return (g.standard_t(d.nu, length) * d.scale).astype(np.float32)
    raise ValueError(d.kind)


def block_bits(w: Workload, i: int, j: int) -> np.ndarray:
    """Bit patterns (uint16 for bf16 / fp16, uint32 for fp32) of block j of tensor i."""
    if w.dtype in FP8_TYPES:
        raise ValueError("FP8 sets are scaled per tensor: use tensor_bits")
    v = block_f32(w, i, j)
    if w.dtype == "fp32":
        return v.view(np.uint32)
    if w.dtype == "fp16":
        return v.astype(np.float16).view(np.uint16)
    return f32_to_bf16_bits(v)


def _fp8_tensor(w: Workload, i: int, threads: int | None) -> np.ndarray:
    import torch
    f = tensor_bits(with_dtype_f32(w), i, threads)  # float32 values as bit patterns
    v = torch.from_numpy(f.view(np.float32))
    dt = getattr(torch, FP8_TYPES[w.dtype])
    amax = float(v.abs().max()) if v.numel() else 1.0
    return (v * (torch.finfo(dt).max / max(amax, 1e-30))).to(dt).view(torch.uint8).numpy()


def with_dtype_f32(w: Workload) -> Workload:
    """The same set as float32 values (the draws before any rounding)."""
    return Workload(w.name, "fp32", w.shapes, w.dist, w.seed, w.note)


def tensor_bits(w: Workload, i: int, threads: int | None = None, out: np.ndarray | None = None):
    """All bit patterns of tensor i (flat)."""
    if w.dtype in FP8_TYPES:
        v = _fp8_tensor(w, i, threads)
        if out is not None:
            out[:] = v
            return out
        return v
    n = w.numels[i]
    dt = np.uint32 if w.dtype == "fp32" else np.uint16
    if out is None:
        out = np.empty(n, dt)
    nblk = (n + GEN_BLOCK - 1) // GEN_BLOCK

    def fill(j):
        s = j * GEN_BLOCK
        b = block_bits(w, i, j)
        out[s:s + b.size] = b

    threads = threads or min(16, os.cpu_count() or 1)
    if nblk == 1 or threads == 1:
        for j in range(nblk):
            fill(j)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def chunk_bits(w: Workload, i: int, k: int, chunk: int = 65536) -> np.ndarray:
    """Elements [k*chunk, (k+1)*chunk) of tensor i, regenerated on their own."""
    n = w.numels[i]
    s = k * chunk
    e = min(n, s + chunk)
    if s >= n:
        raise IndexError("chunk out of range")
    parts = []
    j0, j1 = s // GEN_BLOCK, (e - 1) // GEN_BLOCK
    for j in range(j0, j1 + 1):
        b = block_bits(w, i, j)
        bs = j * GEN_BLOCK
        parts.append(b[max(s, bs) - bs: min(e, bs + b.size) - bs])
    return np.concatenate(parts)


def set_bits(w: Workload, threads: int | None = None):
    """List of flat bit-pattern arrays, one per tensor of the set."""
    return [tensor_bits(w, i, threads) for i in range(len(w.shapes))]
