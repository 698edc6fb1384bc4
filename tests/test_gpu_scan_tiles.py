"""Batches large enough to take the multi-tile path of the encoder's scan and
compaction (more than 4096 chunks: tile sums, per-tile scans, then a
compaction launch), and the two-chunks-per-wavefront decoder on FP32 data,
byte for byte against the oracle: every table, every seek entry, every
payload byte, every raw plane and every decoded element.

Inputs are seeded and synthetic: weight-like chunks (N(0, 0.02) rounded to
BF16, or kept in FP32, and Student-t ones) mixed by chunk index with
chunks of other entropies -- constant (payload of 128 bytes), two-valued
(about one bit per symbol), uniform 16-bit or 32-bit patterns (about eight
bits per coded symbol, so the payload nearly doubles and the decoder's
speculative refills fall behind and take its second pass) and narrow
exponents -- so that chunk sizes jump across every scan-tile boundary.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import lossless_weight_compression_bf16_amd as wc  # noqa: E402
from lossless_weight_compression_bf16_amd import codec, synthetic as S  # noqa: E402

CHUNK = 65536


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    wc.lib()
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _pools(seed, fp32):
    """Value pools the chunks are sliced from (fast to assemble at 10^9
    elements): weight-like, heavy-tailed, uniform bit patterns."""
    g = np.random.default_rng(seed)
    normal = (g.standard_normal(1 << 22) * 0.02).astype(np.float32)
    heavy = (g.standard_t(3.0, 1 << 22) * (0.015 / np.sqrt(3.0))).astype(np.float32)
    if fp32:
        return {"normal": normal.view(np.uint32), "heavy": heavy.view(np.uint32),
                "uniform": g.integers(0, 2 ** 32, 1 << 22, dtype=np.uint64).astype(np.uint32)}
    return {"normal": S.f32_to_bf16_bits(normal), "heavy": S.f32_to_bf16_bits(heavy),
            "uniform": g.integers(0, 2 ** 16, 1 << 22, dtype=np.uint32).astype(np.uint16)}


def _kind(k):
    """The kind of global chunk k (a fixed mix, dense near tile edges too)."""
    if k % 97 == 5:
        return "constant"
    if k % 89 == 7:
        return "uniform"
    if k % 83 == 11:
        return "two"
    if k % 61 == 3:
        return "narrow"
    return "heavy" if k % 7 == 2 else "normal"


def _mixed_batch(ns, seed, fp32=False):
    """Tensors of the given sizes, chunk k of the batch (global index) of
    kind _kind(k)."""
    dt = np.uint32 if fp32 else np.uint16
    pools = _pools(seed, fp32)
    g = np.random.default_rng(seed + 1)
    xs, k = [], 0
    for n in ns:
        x = np.empty(n, dt)
        for c0 in range(0, n, CHUNK):
            m = min(CHUNK, n - c0)
            kind = _kind(k)
            if kind == "constant":
                x[c0:c0 + m] = pools["normal"][k % 1000]
            elif kind == "two":
                pair = pools["normal"][[k % 999, (k * 7 + 3) % 999]]
                x[c0:c0 + m] = pair[g.integers(0, 2, m)]
            elif kind == "narrow":
                # values within one binade: a handful of coded symbols
                x[c0:c0 + m] = pools["normal"][:m] & (0x807FFFFF if fp32 else 0x807F) | (
                    0x3C000000 if fp32 else 0x3C00)
            else:
                pool = pools[kind]
                s = int(g.integers(0, pool.size - m + 1))
                x[c0:c0 + m] = pool[s:s + m]
            k += 1
        xs.append(x)
    return xs


def _check_batch(xs, dtype, dev, oracle_lib, what):
    ity, nty = (torch.int32, np.int32) if dtype == "fp32" else (torch.int16, np.int16)
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    ts = [torch.from_numpy(x.view(nty)).to(dev).view(tdt) for x in xs]
    chunks = sum(-(-x.size // CHUNK) for x in xs)
    _say(f"[tiles] {what}: {len(xs)} tensors, {sum(x.size for x in xs)} elements, {chunks} chunks")
    e = codec.encode_batch(ts)
    o = oracle_lib.encode_batch(xs, dtype, threads=16)
    assert np.array_equal(e.tables.cpu().numpy().view("<u2").reshape(-1), o.tables.reshape(-1)), f"{what}: tables"
    assert np.array_equal(e.seek.cpu().numpy().view("<u8"), o.seek), f"{what}: seek"
    assert np.array_equal(e.payload.cpu().numpy(), o.payload), f"{what}: payload"
    assert np.array_equal(e.raw.cpu().numpy(), o.raw), f"{what}: raw planes"
    _say(f"[tiles] {what}: tables, seek, payload and raw planes equal to the oracle "
         f"(payload {o.payload.size} B)")
    outs = codec.decode_batch(e)
    for t, y in zip(ts, outs):
        assert torch.equal(t.view(ity), y.view(ity)), f"{what}: decode"
    _say(f"[tiles] {what}: decoded bit for bit")
    return e, o


def test_many_small_tensors_span_three_scan_tiles(dev, oracle_lib):
    """8,194 tensors of 1 to 70,000 elements, 8,195 chunks (an odd count
    above two scan tiles, ragged tails everywhere, zeroed gaps between raw
    planes): the scan and compaction across tiles of small payloads."""
    g = np.random.default_rng(21)
    ns = [int(v) for v in g.integers(1, 3000, 8194)]
    ns[100] = 70000          # a two-chunk tensor
    ns[5000] = CHUNK         # exactly one full chunk
    xs = _mixed_batch(ns, 22)
    assert sum(-(-n // CHUNK) for n in ns) % 2 == 1
    e, o = _check_batch(xs, "bf16", dev, oracle_lib, "8194 small tensors")
    assert e.seek.numel() - 1 > 2 * 4096


def test_full_chunks_span_three_scan_tiles(dev, oracle_lib):
    """8,297 chunks of up to 65,536 symbols in three tensors with ragged
    tails, kinds mixed by chunk index: the multi-tile scan and compaction
    at full chunk size, and the two-chunk decoder over it."""
    ns = [4096 * CHUNK + 12345, 3000 * CHUNK + 1, 1198 * CHUNK + 40000]
    xs = _mixed_batch(ns, 23)
    chunks = sum(-(-n // CHUNK) for n in ns)
    assert chunks == 8297 and chunks % 2 == 1
    e, o = _check_batch(xs, "bf16", dev, oracle_lib, "8297 full chunks")
    sizes = np.diff(o.seek.astype(np.int64))
    assert sizes.min() == 128 and sizes.max() > 65536  # constant and uniform chunks present


def test_fp32_two_chunk_decoder(dev, oracle_lib):
    """FP32 past the one-chunk-per-wavefront limit (2,101 chunks, odd, with a
    ragged tail, an empty and a one-element tensor): the exponent plane
    through the two-chunk decoder, the sign / mantissa planes joined inside
    its pipelined loop, and chunks of uniform 32-bit patterns (8 bits per
    coded symbol) that outrun the speculative refills and are decoded a
    second time."""
    from lossless_weight_compression_bf16_amd import _binding as B
    ns = [2048 * CHUNK + 777, 0, 1, 51 * CHUNK]
    xs = _mixed_batch(ns, 24, fp32=True)
    chunks = sum(-(-n // CHUNK) for n in ns)
    assert chunks == 2101
    e, o = _check_batch(xs, "fp32", dev, oracle_lib, "fp32 2101 chunks")
    one, dwords = B.wc_decode_variant("fp32", chunks, sum(ns), o.payload.size)
    assert not one and dwords == 1  # two chunks per wavefront, one-dword refills
    sizes = np.diff(o.seek.astype(np.int64))
    assert sizes.max() > 2 * 64 * (CHUNK // 256)  # chunks above 64 words per 8-step group exist
