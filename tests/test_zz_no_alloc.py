"""wc_encode_noalloc (the encoder on the library's fixed device scratch)
against wc_encode with a scratch buffer from the caller: identical tables,
seek table, payload and raw planes, and a bit-exact decode, on calls in a
row whose inputs shrink (so the second call runs over what the first left
in the shared array), plus an FP32 call with a tensor-wide table and
CRC-32s, and the host-side refusal of a tensor past the array's size.
All calls go through the C ABI."""
import ctypes
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import lossless_weight_compression_bf16_amd as wc  # noqa: E402
from lossless_weight_compression_bf16_amd import _binding as B, codec, synthetic as S  # noqa: E402


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    wc.lib()
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _buffers(lay, dev, crc):
    raw = torch.zeros(max(lay.raw_bytes, 16), dtype=torch.uint8, device=dev)
    tables = torch.zeros(max(lay.table_bytes // 2, 8), dtype=torch.int16, device=dev)
    seek = torch.zeros(lay.num_chunks + 1, dtype=torch.int64, device=dev)
    payload = torch.zeros(max(lay.payload_capacity, 16), dtype=torch.uint8, device=dev)
    c = torch.zeros(max(lay.num_chunks, 1), dtype=torch.int32, device=dev) if crc else None
    return raw, tables, seek, payload, c


def _encode_both(x, fmt, dev, crc=False):
    lay = B.wc_query_layout(fmt, x.numel())
    a = _buffers(lay, dev, crc)
    b = _buffers(lay, dev, crc)
    scratch = torch.empty(max(lay.scratch_bytes, 256), dtype=torch.uint8, device=dev)
    err_a = torch.zeros(1, dtype=torch.int32, device=dev)
    err_b = torch.zeros(1, dtype=torch.int32, device=dev)
    B.wc_encode(fmt, x, x.numel(), B.make_buffers(*a[:4], lay.payload_capacity, a[4]), scratch, scratch.numel(),
                err_a)
    B.wc_encode_noalloc(fmt, x, x.numel(), B.make_buffers(*b[:4], lay.payload_capacity, b[4]), err_b)
    torch.cuda.synchronize()
    assert int(err_a.item()) == 0 and int(err_b.item()) == 0
    total = int(a[2][-1].item())
    assert int(b[2][-1].item()) == total
    for name, u, v in zip(("raw", "tables", "seek"), a[:3], b[:3]):
        assert torch.equal(u, v), name
    assert torch.equal(a[3][:total], b[3][:total]), "payload"
    if crc:
        assert torch.equal(a[4], b[4]), "crc"
    return lay, b, total


@pytest.mark.parametrize("first", [True, False])
def test_noalloc_matches_wc_encode(dev, first):
    """Calls in a row, each smaller than the one before, on the same shared
    array (run twice: the second pass starts over what the first left)."""
    w = S.workload("llama3-8b-bf16")
    big = S.chunk_bits(w, 0, 0, chunk=9 * 65536 + 4321)
    cases = [("bf16", big), ("bf16", big[: 3 * 65536 + 77]), ("bf16", big[5:6])]
    if not first:
        cases = cases[1:] + cases[:1]
    for dtype, bits in cases:
        x = torch.from_numpy(bits.view(np.int16)).to(dev)
        lay, b, total = _encode_both(x, B.format_word(dtype), dev)
        e = codec.Encoded(dtype, x.numel(), (x.numel(),), torch.bfloat16, b[0][: lay.raw_bytes],
                          b[1][: lay.table_bytes // 2], b[2], b[3][:total])
        y = codec.decode(e)
        assert torch.equal(y.view(torch.int16), x), dtype
        _say(f"[noalloc] {dtype} n={x.numel()}: same bytes as wc_encode, decoded bit for bit")


def test_noalloc_fp32_tensor_table_crc(dev):
    g = np.random.default_rng(31)
    bits = (g.standard_normal(2 * 65536 + 999) * 0.02).astype(np.float32).view(np.int32)
    x = torch.from_numpy(bits).to(dev)
    fmt = B.format_word("fp32", tensor_table=True, crc=True)
    _encode_both(x, fmt, dev, crc=True)
    _say("[noalloc] fp32 with a tensor-wide table and CRC-32s: same bytes as wc_encode")


def test_noalloc_refuses_more_than_its_array(dev):
    L = B.lib()
    for fmt in (B.format_word("bf16"), B.format_word("fp32", tensor_table=True)):
        c = B.wc_noalloc_max_chunks(fmt)
        assert c >= 1000 and B.wc_query_layout(fmt, c * 65536).scratch_bytes <= B.WC_NOALLOC_SCRATCH_BYTES
        assert B.wc_query_layout(fmt, (c + 1) * 65536).scratch_bytes > B.WC_NOALLOC_SCRATCH_BYTES
        # refused on the host before any pointer is used or anything enqueued
        bufs = B.wc_buffers(0, 0, 0, 0, 0)
        rc = L.wc_encode_noalloc(fmt, 0x1000, (c + 1) * 65536, ctypes.byref(bufs), None, None)
        assert rc == B.WC_ERR_CAPACITY
