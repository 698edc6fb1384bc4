"""Decode fused with its consumer (Y += X W^T from compressed BF16 weights)
through the C ABI, against the oracle.

Checked per case: the GPU's tile order equals the oracle's element by
element (both directions); the bytes encoded from it equal the oracle's
encoding of the oracle's tile order; the weights decode back bit for bit;
and Y equals the oracle's double-precision X W^T within the rounding bound
of fp32 accumulation of exact BF16 products: |Y - Y_ref| <= (k + 16) 2^-24
sum_t |x_t w_t| (plus the initial Y's own rounding when Y starts non-zero).
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import lossless_weight_compression_bf16_amd as wc  # noqa: E402
from lossless_weight_compression_bf16_amd import _binding as B, codec, gemm as G, synthetic as S  # noqa: E402


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    wc.lib()
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _wbits(rows, cols, seed, sigma=0.02):
    g = np.random.default_rng(seed)
    return S.f32_to_bf16_bits((g.standard_normal(rows * cols) * sigma).astype(np.float32)).reshape(rows, cols)


def _xbits(m, cols, seed):
    g = np.random.default_rng(1000 + seed)
    return S.f32_to_bf16_bits(g.standard_normal(m * cols).astype(np.float32)).reshape(m, cols)


def _dev16(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def _run(shapes, m, dev, oracle_lib, what, reorder=False, tensor_table=False, crc=False, y0=False, seed=0):
    _say(f"[gemm] {what}: shapes={shapes} m={m} reorder={reorder} tt={tensor_table} crc={crc} y0={y0}")
    wb = [_wbits(r, c, seed + i) for i, (r, c) in enumerate(shapes)]
    xb = [_xbits(m, c, seed + i) for i, (r, c) in enumerate(shapes)]
    ws = [_dev16(w, dev) for w in wb]
    xs = [_dev16(x, dev) for x in xb]
    # tile order, both directions, against the oracle
    tiles_o = [oracle_lib.tile_order(w) for w in wb]
    for w, t_o, (r, c) in zip(ws, tiles_o, shapes):
        t = G.to_tiles(w)
        assert np.array_equal(t.view(torch.int16).cpu().numpy().view(np.uint16), t_o), f"{what}: tile order"
        back = G.from_tiles(t, r, c)
        assert torch.equal(back.view(torch.int16), w.view(torch.int16)), f"{what}: inverse tile order"
    e = G.encode_weights(ws, reorder=reorder, tensor_table=tensor_table, crc=crc)
    layout = "bf16r" if reorder else "bf16"
    opts = (0x100 if tensor_table else 0) | (0x400 if crc else 0)
    o = oracle_lib.encode_batch(tiles_o, layout, threads=16, opts=opts)
    assert np.array_equal(e.batch.seek.cpu().numpy().view(np.uint64), o.seek), f"{what}: seek"
    assert np.array_equal(e.batch.payload.cpu().numpy(), o.payload), f"{what}: payload"
    assert np.array_equal(e.batch.tables.cpu().numpy().view(np.uint16).reshape(-1), o.tables.reshape(-1)), what
    for w, d in zip(ws, G.decode_weights(e)):
        assert torch.equal(d.view(torch.int16), w.view(torch.int16)), f"{what}: decoded weights"
    ys = None
    base = []
    if y0:
        g = np.random.default_rng(99)
        base = [g.standard_normal((m, r)).astype(np.float32) for r, _ in shapes]
        ys = [torch.from_numpy(b).to(dev) for b in base]
    ys = G.decode_gemm(e, xs, ys)
    torch.cuda.synchronize()
    for i, ((r, c), y) in enumerate(zip(shapes, ys)):
        ref, mag = oracle_lib.gemm_bf16(xb[i], wb[i], magnitude=True)
        got = y.cpu().numpy().astype(np.float64)
        bound = (c + 16) * 2.0 ** -24 * mag + 1e-30
        if y0:
            ref = ref + base[i].astype(np.float64)
            bound = bound + 2.0 ** -24 * np.abs(ref)
        err = np.abs(got - ref)
        worst = np.unravel_index(np.argmax(err - bound), err.shape)
        assert np.all(err <= bound), (f"{what}: matrix {i} ({r}x{c}) at {worst}: got {got[worst]!r} "
                                      f"want {ref[worst]!r} bound {bound[worst]!r}")
    return e


def test_one_tile_one_row(dev, oracle_lib):
    _run([(16, 16)], 1, dev, oracle_lib, "one tile, m=1")


def test_two_panels_per_chunk(dev, oracle_lib):
    _run([(64, 2048)], 16, dev, oracle_lib, "64x2048, m=16")


def test_moe_w2_shape(dev, oracle_lib):
    _run([(7168, 2048)], 16, dev, oracle_lib, "expert w2 7168x2048, m=16")


def test_panels_across_chunks(dev, oracle_lib):
    # 257 tiles per panel: panels cross chunk boundaries, Y gets atomics from two chunks
    _run([(48, 4112)], 5, dev, oracle_lib, "48x4112, m=5")


def test_many_panels_per_chunk(dev, oracle_lib):
    # 48 tiles per panel: a chunk touches up to 7 panels
    _run([(96, 768), (32, 3072)], 16, dev, oracle_lib, "gpt2 shapes, m=16")


@pytest.mark.parametrize("m", [17, 32, 33, 64])
def test_row_blocks(dev, oracle_lib, m):
    _run([(96, 2048), (16, 4096), (32, 6144)], m, dev, oracle_lib, f"three shapes, m={m}", seed=m)


def test_odd_chunk_count_and_mixed_lengths(dev, oracle_lib):
    # 1 + 2 + 1 chunks: waves pair a one-tile chunk with a full one; the last wave's second half shadows
    _run([(16, 16), (64, 2048), (32, 80)], 3, dev, oracle_lib, "mixed lengths, odd count")


def test_options(dev, oracle_lib):
    _run([(128, 2048), (16, 4096)], 16, dev, oracle_lib, "reorder", reorder=True)
    _run([(128, 2048), (16, 4096)], 16, dev, oracle_lib, "tensor table + crc", tensor_table=True, crc=True)


def test_accumulates_into_y(dev, oracle_lib):
    _run([(64, 2048)], 8, dev, oracle_lib, "Y += X W^T", y0=True)


def test_corrupt_table_is_reported(dev, oracle_lib):
    w = _dev16(_wbits(64, 2048, 5), dev)
    e = G.encode_weights([w])
    e.batch.tables[1, 0] += 1  # chunk 1's table no longer sums to 4096
    x = _dev16(_xbits(4, 2048, 5), dev)
    with pytest.raises(B.WcError, match="bad table"):
        G.decode_gemm(e, [x])


def test_crc_mismatch_is_reported(dev, oracle_lib):
    w = _dev16(_wbits(64, 2048, 6), dev)
    e = G.encode_weights([w], crc=True)
    e.batch.crc[0] ^= 1
    x = _dev16(_xbits(4, 2048, 6), dev)
    with pytest.raises(B.WcError, match="CRC mismatch"):
        G.decode_gemm(e, [x])


def test_rejected_arguments(dev):
    w = _dev16(_wbits(256, 768, 1), dev)
    e = G.encode_weights([w])
    x64 = _dev16(_xbits(64, 768, 1), dev)
    with pytest.raises(B.WcError):  # a full chunk spans 6 panels: more than 64 rows leave accumulators for
        G.decode_gemm(e, [x64])
    x65 = _dev16(_xbits(65, 768, 1), dev)
    with pytest.raises(B.WcError):
        G.decode_gemm(e, [x65])
    e2 = G.EncodedWeights(codec.encode_batch([G.to_tiles(w)], raw_fallback=True), e.shapes)
    with pytest.raises(B.WcError):
        G.decode_gemm(e2, [_dev16(_xbits(4, 768, 1), dev)])
    with pytest.raises(ValueError):
        G.to_tiles(torch.zeros((24, 16), dtype=torch.bfloat16, device=dev))
