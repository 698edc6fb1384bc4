"""GPU path of the FP8 layouts against the oracle, byte for byte.

FP8 E4M3 and E5M2 ("PTWM" README: bit reorder into the high nibble, 2-plane
nibble split): tables, seek table, payload and the packed raw nibbles must
equal the oracle's, and the decoded bytes the input, through both decoder
variants and with the format options.  Tensors are uint8 bit patterns given
an explicit layout; all calls go through the C ABI.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import lossless_weight_compression_bf16_amd as wc  # noqa: E402
from lossless_weight_compression_bf16_amd import _binding as B, codec  # noqa: E402

TT, RF = 0x100, 0x200
FP8 = {"fp8e4m3": torch.float8_e4m3fn, "fp8e5m2": torch.float8_e5m2}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    wc.lib()
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _weights(layout, n, seed):
    """Gaussian draws scaled so the largest magnitude is the format's largest
    finite value, rounded by torch on the CPU."""
    if n == 0:
        return np.zeros(0, np.uint8)
    x = torch.from_numpy(np.random.default_rng(seed).standard_normal(n).astype(np.float32))
    dt = FP8[layout]
    return (x * (torch.finfo(dt).max / max(float(x.abs().max()), 1e-30))).to(dt).view(torch.uint8).numpy()


def _upload(o, layout, opts, dev):
    def t(a, dt):
        a = np.ascontiguousarray(a)
        if a.size == 0:
            a = np.zeros(16 // np.dtype(dt).itemsize, dt)
        return torch.from_numpy(a.view(dt)).to(dev)
    return codec.Encoded(layout, o.n, (o.n,), torch.uint8, t(o.raw, np.uint8)[: o.raw.size],
                         t(o.tables.reshape(-1), np.int16)[: o.tables.size], t(o.seek, np.int64),
                         t(o.payload, np.uint8)[: o.payload.size], B.format_word(layout) | opts)


def _one(layout, opts, x, dev, oracle_lib, what):
    _say(f"[fp8] {what}: layout={layout} opts={opts:#x} n={x.size}")
    xt = torch.from_numpy(np.ascontiguousarray(x, np.uint8)).to(dev)
    e = codec.encode(xt, layout=layout, tensor_table=bool(opts & TT), raw_fallback=bool(opts & RF))
    o = oracle_lib.encode(x, layout, threads=16, opts=opts)
    h = e.to_host()
    assert np.array_equal(h["tables"].reshape(-1), o.tables.reshape(-1)), f"{what}: tables"
    assert np.array_equal(h["seek"], o.seek), f"{what}: seek"
    assert np.array_equal(h["payload"], o.payload), f"{what}: payload"
    assert np.array_equal(h["raw"], o.raw), f"{what}: raw nibbles"
    y = codec.decode(e)
    assert torch.equal(y.cpu(), xt.cpu()), f"{what}: decode"
    z = codec.decode(_upload(o, layout, opts, dev))
    assert torch.equal(z.cpu(), xt.cpu()), f"{what}: decode of oracle bytes"
    return e, o


@pytest.mark.parametrize("layout", ["fp8e4m3", "fp8e5m2"])
@pytest.mark.parametrize("n", [1, 2, 5, 15, 17, 33, 65535, 65536, 65537, 3 * 65536 + 12345])
def test_fp8_sizes(dev, oracle_lib, layout, n):
    _one(layout, 0, _weights(layout, n, n), dev, oracle_lib, f"{layout} n={n}")


@pytest.mark.parametrize("layout", ["fp8e4m3", "fp8e5m2"])
def test_fp8_every_pattern(dev, oracle_lib, layout):
    g = np.random.default_rng(3)
    x = np.concatenate([g.permutation(np.tile(np.arange(256, dtype=np.uint8), 300)),
                        np.arange(256, dtype=np.uint8), g.integers(0, 256, 1001).astype(np.uint8)])
    _one(layout, 0, x, dev, oracle_lib, f"{layout} all patterns")


@pytest.mark.parametrize("layout", ["fp8e4m3", "fp8e5m2"])
def test_fp8_two_chunk_wavefronts(dev, oracle_lib, layout):
    n = 2401 * 65536 - 333
    _one(layout, 0, _weights(layout, n, 4), dev, oracle_lib, f"{layout} 2401 chunks")


@pytest.mark.parametrize("opts", [TT, RF, TT | RF])
def test_fp8_options(dev, oracle_lib, opts):
    g = np.random.default_rng(5)
    parts = [_weights("fp8e4m3", 65536, 6), g.integers(0, 256, 65536).astype(np.uint8),
             _weights("fp8e4m3", 2 * 65536, 7), g.integers(0, 256, 9).astype(np.uint8)]
    _one("fp8e4m3", opts, np.concatenate(parts), dev, oracle_lib, f"fp8 options {opts:#x}")


def test_fp8_batch(dev, oracle_lib):
    xs = [_weights("fp8e5m2", n, i) for i, n in enumerate([70001, 0, 65536, 3, 2 * 65536 + 1])]
    _say("[fp8] batch e5m2")
    ts = [torch.from_numpy(x).to(dev) if x.size else torch.empty(0, dtype=torch.uint8, device=dev) for x in xs]
    e = codec.encode_batch(ts, layout="fp8e5m2")
    o = oracle_lib.encode_batch(xs, "fp8e5m2", threads=8)
    assert np.array_equal(e.tables.cpu().numpy().view(np.uint16).reshape(-1), o.tables.reshape(-1))
    assert np.array_equal(e.seek.cpu().numpy().view(np.uint64), o.seek)
    assert np.array_equal(e.payload.cpu().numpy(), o.payload)
    assert np.array_equal(e.raw.cpu().numpy(), o.raw)
    for x, y in zip(xs, codec.decode_batch(e)):
        assert np.array_equal(y.cpu().numpy(), x)
