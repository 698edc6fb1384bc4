"""GPU path of the format variants against the oracle, byte for byte.

Layouts BF16_REORDER, FP16, FP16_REORDER (the PTWM README's bit reorder and
2-plane split) and the options TENSOR_TABLE and RAW_FALLBACK: tables, seek
table, payload and raw planes must equal the oracle's, and the decoded bit
patterns the input, through both decoder variants (one chunk per wavefront
while every chunk fits on a 256-CU device at once: up to 2,048 chunks with
one-dword refills, 1,792 with two-dword ones; two chunks per wavefront
above).  All calls go through the C ABI.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import lossless_weight_compression_bf16_amd as wc  # noqa: E402
from lossless_weight_compression_bf16_amd import _binding as B, codec, synthetic as S  # noqa: E402

TT = 0x100
RF = 0x200
TORCH_OF = {"bf16": torch.bfloat16, "bf16r": torch.bfloat16, "fp16": torch.float16, "fp16r": torch.float16,
            "fp32": torch.float32}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    wc.lib()
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bits_of(layout, x):
    return np.ascontiguousarray(x).view(np.uint32 if layout == "fp32" else np.uint16)


def _tensor(layout, x, dev):
    a = _bits_of(layout, x)
    t = torch.from_numpy(a.view(np.int32 if layout == "fp32" else np.int16)).to(dev)
    return t.view(TORCH_OF[layout])


def _weights16(layout, n, seed, sigma=0.02):
    g = np.random.default_rng(seed)
    f = (g.standard_normal(n) * sigma).astype(np.float32)
    if layout.startswith("fp16"):
        return f.astype(np.float16).view(np.uint16)
    return S.f32_to_bf16_bits(f)


def _compare(e, o, what):
    h = e.to_host()
    assert np.array_equal(h["tables"].reshape(-1), o.tables.reshape(-1)), f"{what}: tables"
    assert np.array_equal(h["seek"], o.seek), f"{what}: seek"
    assert np.array_equal(h["payload"], o.payload), f"{what}: payload"
    assert np.array_equal(h["raw"], o.raw), f"{what}: raw planes"


def _upload(o, layout, opts, dev):
    def t(a, dt):
        a = np.ascontiguousarray(a)
        if a.size == 0:
            a = np.zeros(16 // np.dtype(dt).itemsize, dt)
        return torch.from_numpy(a.view(dt)).to(dev)
    return codec.Encoded(layout, o.n, (o.n,), TORCH_OF[layout], t(o.raw, np.uint8)[: o.raw.size],
                         t(o.tables.reshape(-1), np.int16)[: o.tables.size], t(o.seek, np.int64),
                         t(o.payload, np.uint8)[: o.payload.size], B.format_word(layout) | opts)


def _one(layout, opts, x, dev, oracle_lib, what):
    _say(f"[variants] {what}: layout={layout} opts={opts:#x} n={x.size}")
    xt = _tensor(layout, x, dev)
    base = layout[:4]
    e = codec.encode(xt, reorder=layout.endswith("r"), tensor_table=bool(opts & TT),
                     raw_fallback=bool(opts & RF))
    assert e.dtype == layout
    o = oracle_lib.encode(_bits_of(layout, x), layout, threads=16, opts=opts)
    _compare(e, o, what)
    ity = torch.int32 if base == "fp32" else torch.int16
    ref = xt.view(ity).cpu()
    y = codec.decode(e)
    assert torch.equal(y.view(ity).cpu(), ref), f"{what}: decode"
    z = codec.decode(_upload(o, layout, opts, dev))
    assert torch.equal(z.view(ity).cpu(), ref), f"{what}: decode of oracle bytes"
    return e, o


LAYOUTS16 = ["bf16r", "fp16", "fp16r"]


@pytest.mark.parametrize("layout", LAYOUTS16)
@pytest.mark.parametrize("n", [1, 33, 65536, 3 * 65536 + 12345])
def test_layout_sizes(dev, oracle_lib, layout, n):
    _one(layout, 0, _weights16(layout, n, n), dev, oracle_lib, f"{layout} n={n}")


@pytest.mark.parametrize("layout", LAYOUTS16)
def test_layout_every_pattern(dev, oracle_lib, layout):
    v = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    g = np.random.default_rng(5)
    x = np.concatenate([g.permutation(v), v, g.permutation(v)[:40001]])
    _one(layout, 0, x, dev, oracle_lib, f"{layout} all patterns")


@pytest.mark.parametrize("layout", ["bf16r", "fp16r"])
def test_layout_two_chunk_wavefronts(dev, oracle_lib, layout):
    """More than 2,048 chunks: the two-chunks-per-wavefront decoder, whose
    pipelined store path applies the inverse bit reorder."""
    n = 2401 * 65536 - 999
    _one(layout, 0, _weights16(layout, n, 7), dev, oracle_lib, f"{layout} 2401 chunks")


@pytest.mark.parametrize("layout", ["bf16", "bf16r", "fp16", "fp32"])
def test_tensor_table(dev, oracle_lib, layout):
    n = 9 * 65536 + 777
    if layout == "fp32":
        x = (np.random.default_rng(8).standard_normal(n) * 0.02).astype(np.float32).view(np.uint32)
    else:
        x = _weights16(layout, n, 8)
    e, o = _one(layout, TT, x, dev, oracle_lib, f"{layout} tensor table")
    assert tuple(e.tables.shape) == (1, 256)


def test_tensor_table_of_mixed_chunks(dev, oracle_lib):
    """Chunks with different supports (the table must cover every symbol of
    the tensor), a chunk of one symbol, and a short tail."""
    g = np.random.default_rng(9)
    parts = [_weights16("bf16", 65536, 1, 0.001), _weights16("bf16", 65536, 2, 0.5),
             np.full(65536, 0x3F80, np.uint16), _weights16("bf16", 65536, 3, 30.0),
             g.integers(0, 65536, 501).astype(np.uint16)]
    _one("bf16", TT, np.concatenate(parts), dev, oracle_lib, "tensor table, mixed chunks")


def _uniform_chunk(seed):
    g = np.random.default_rng(seed)
    hi = g.permutation(np.repeat(np.arange(256, dtype=np.uint16), 256))
    return (hi << 8) | g.integers(0, 256, 65536).astype(np.uint16)


def test_raw_fallback(dev, oracle_lib):
    parts = [_weights16("bf16", 65536, 1), _uniform_chunk(2), _uniform_chunk(3), _weights16("bf16", 65536, 4),
             _uniform_chunk(5)[:70]]
    x = np.concatenate(parts)
    e, o = _one("bf16", RF, x, dev, oracle_lib, "raw fallback")
    sizes = np.diff(o.seek.astype(np.int64))
    assert list(sizes[1:3]) == [65536, 65536] and sizes[4] == 72 and sizes[0] < 65536


@pytest.mark.parametrize("opts", [RF, TT | RF])
def test_raw_fallback_two_chunk_wavefronts(dev, oracle_lib, opts):
    """2,101 chunks, every seventh one uniform (stored raw), so raw and coded
    chunks share wavefronts in both orders, plus a raw short tail."""
    g = np.random.default_rng(12)
    n_chunks = 2101
    x = _weights16("bf16", n_chunks * 65536, 13)
    for k in range(0, n_chunks - 1, 7):
        x[k * 65536:(k + 1) * 65536] = _uniform_chunk(k)
    x = np.concatenate([x, g.integers(0, 65536, 5).astype(np.uint16)])
    e, o = _one("bf16r", opts, x, dev, oracle_lib, f"raw fallback 2102 chunks opts={opts:#x}")
    raw_chunks = int((np.diff(o.seek.astype(np.int64))[:-1] == 65536).sum())
    assert raw_chunks == len(range(0, n_chunks - 1, 7))


def test_raw_fallback_fp32_with_tensor_table(dev, oracle_lib):
    g = np.random.default_rng(14)
    n = 4 * 65536 + 3
    u = g.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    u[65536:2 * 65536] = (g.standard_normal(65536) * 0.02).astype(np.float32).view(np.uint32)
    _one("fp32", TT | RF, u, dev, oracle_lib, "fp32 raw fallback + tensor table")


def test_raw_chunk_bad_padding_is_flagged(dev, oracle_lib):
    x = np.concatenate([_weights16("bf16", 65536, 15), _uniform_chunk(16)[:6]])
    o = oracle_lib.encode(x, "bf16", opts=RF)
    assert int(o.seek[2] - o.seek[1]) == 8
    o.payload = o.payload.copy()
    o.payload[-1] = 7
    _, bits_or = oracle_lib.decode(o, strict=False)
    assert bits_or & oracle_lib.EF_BAD_TAIL
    e = _upload(o, "bf16", RF, dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.empty(x.size, dtype=torch.int16, device=dev)
    B.wc_decode(e.fmt, e.buffers(), e.n, out, err)
    torch.cuda.synchronize()
    assert int(err.item()) == bits_or


def test_batch_with_options(dev, oracle_lib):
    """Tensors with tensor tables and raw fallback in one launch sequence,
    empty and tiny tensors included."""
    xs = [_weights16("bf16", 70000, 21), np.zeros(0, np.uint16), _uniform_chunk(22), _weights16("bf16", 3, 23),
          _weights16("bf16", 2 * 65536, 24)]
    for layout in ("bf16", "bf16r"):
        opts = TT | RF
        _say(f"[variants] batch {layout} opts={opts:#x}")
        ts = [_tensor(layout, x, dev) for x in xs]
        e = codec.encode_batch(ts, reorder=layout.endswith("r"), tensor_table=True, raw_fallback=True)
        o = oracle_lib.encode_batch([_bits_of(layout, x) for x in xs], layout, threads=8, opts=opts)
        assert tuple(e.tables.shape) == (len(xs), 256)
        assert np.array_equal(e.tables.cpu().numpy().view(np.uint16).reshape(-1), o.tables.reshape(-1))
        assert np.array_equal(e.seek.cpu().numpy().view(np.uint64), o.seek)
        assert np.array_equal(e.payload.cpu().numpy(), o.payload)
        assert np.array_equal(e.raw.cpu().numpy(), o.raw)
        ys = codec.decode_batch(e)
        for x, y in zip(xs, ys):
            assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), x)


def test_empty_tensor_with_tensor_table(dev):
    e = codec.encode(torch.empty(0, dtype=torch.bfloat16, device=dev), tensor_table=True)
    assert tuple(e.tables.shape) == (1, 256) and not e.tables.cpu().numpy().any()



def test_wide_refills_with_uniform_chunks(dev, oracle_lib):
    """FP16 weights (about 5.5 bits per coded byte) select the two-dword
    refills; every fifth chunk has uniform coded bytes (8 bits: 128 words per
    group, the refills' full rate), so some groups outrun the landed words
    and their chunk is decoded a second time; 2,401 chunks put them in
    two-chunk wavefronts next to ordinary ones, and short chunks at the end
    clamp the paired loads at the stream end."""
    g = np.random.default_rng(31)
    n_chunks = 2401
    x = _weights16("fp16", n_chunks * 65536, 32)
    for k in range(0, n_chunks, 5):
        hi = g.permutation(np.repeat(np.arange(256, dtype=np.uint16), 256))
        x[k * 65536:(k + 1) * 65536] = (hi << 8) | g.integers(0, 256, 65536).astype(np.uint16)
    x = np.concatenate([x, _weights16("fp16", 77, 33)])
    _one("fp16", 0, x, dev, oracle_lib, "fp16 2402 chunks, uniform every fifth")


def test_crc32_table(dev, oracle_lib):
    """The CRC option: crc[k] equals the oracle's CRC-32 of chunk k's payload
    (and zlib's), over chunks of every kind: weights, a raw one, a tail of 70
    symbols, and a one-symbol chunk whose payload is the 128 bytes of states."""
    import zlib
    parts = [_weights16("bf16", 65536, 51), _uniform_chunk(52), _weights16("bf16", 3 * 65536, 53),
             np.full(65536, 0x3F80, np.uint16), _uniform_chunk(54)[:70]]
    x = np.concatenate(parts)
    xt = _tensor("bf16", x, dev)
    e = codec.encode(xt, raw_fallback=True, crc=True)
    h = e.to_host()
    want = oracle_lib.chunk_crc(h["seek"], h["payload"])
    assert np.array_equal(h["crc"], want)
    for k in (0, 1, 6):
        assert int(h["crc"][k]) == zlib.crc32(h["payload"][int(h["seek"][k]):int(h["seek"][k + 1])].tobytes())
    y = codec.decode(e)
    assert torch.equal(y.view(torch.int16).cpu(), xt.view(torch.int16).cpu())


def test_crc32_detects_a_flipped_byte(dev, oracle_lib):
    x = _weights16("bf16", 5 * 65536 + 9, 55)
    o = oracle_lib.encode(x, "bf16", opts=RF)
    crc = oracle_lib.chunk_crc(o.seek, o.payload)
    for k in (0, 3, 5):
        bad = o.payload.copy()
        pos = int(o.seek[k]) + (int(o.seek[k + 1] - o.seek[k]) // 2 & ~3) + 1
        bad[pos] ^= 0x10
        e = _upload(oracle_lib.Encoded(o.dtype, o.n, o.raw, o.tables, o.seek, bad, RF), "bf16", RF | 0x400, dev)
        e.crc = torch.from_numpy(crc.view(np.int32)).to(dev)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        out = torch.empty(x.size, dtype=torch.int16, device=dev)
        B.wc_decode(e.fmt, e.buffers(), e.n, out, err)
        torch.cuda.synchronize()
        assert int(err.item()) & B.EF_BAD_CRC, k
    good = _upload(o, "bf16", RF | 0x400, dev)
    good.crc = torch.from_numpy(crc.view(np.int32)).to(dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.empty(x.size, dtype=torch.int16, device=dev)
    B.wc_decode(good.fmt, good.buffers(), good.n, out, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert np.array_equal(out.cpu().numpy().view(np.uint16), x)


def test_crc32_batch(dev, oracle_lib):
    xs = [_weights16("bf16", n, 60 + i) for i, n in enumerate([70000, 0, 65536, 3, 2 * 65536])]
    ts = [_tensor("bf16", x, dev) for x in xs]
    e = codec.encode_batch(ts, crc=True, tensor_table=True)
    seek = e.seek.cpu().numpy().view(np.uint64)
    assert np.array_equal(e.crc.cpu().numpy().view(np.uint32), oracle_lib.chunk_crc(seek, e.payload.cpu().numpy()))
    for x, y in zip(xs, codec.decode_batch(e)):
        assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), x)
