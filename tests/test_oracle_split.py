"""Pins of the oracle's plane split against numpy's own view of the bytes.

The split is the byte-plane transform of the weight-compression (Split12)
README (BF16: high byte coded, low byte raw) and the SMEF README's pass 3
(FP32 sign / exponent / mantissa streams).  numpy's little-endian byte view
and np.packbits are independent of the oracle's shifts and masks.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def test_bf16_split_exhaustive(oracle_lib):
    o = oracle_lib
    v = np.arange(65536, dtype=np.uint16)
    hi, lo = o.split_bf16(v)
    b = v.view(np.uint8)  # little endian: low byte first
    assert np.array_equal(lo, b[0::2])
    assert np.array_equal(hi, b[1::2])
    assert np.array_equal(o.merge_bf16(hi, lo), v)
    # shuffled, in several sizes (including ones that are not multiples of 8)
    g = np.random.default_rng(1)
    for n in (1, 7, 33, 1000, 65537):
        x = g.permutation(65536 * 2)[:n].astype(np.uint32).astype(np.uint16)
        h, l = o.split_bf16(x)
        assert np.array_equal(o.merge_bf16(h, l), x)
        assert np.array_equal(h, x.view(np.uint8)[1::2])


def test_bf16_split_semantics():
    """hi holds the sign and exponent bits 7..1 of real bf16 values."""
    import torch
    vals = torch.tensor([1.0, -1.0, 2.0, 0.5, -0.0, float("inf")], dtype=torch.bfloat16)
    u = vals.view(torch.uint16).numpy()
    hi = u >> 8
    # 1.0 = 0x3F80: sign 0, exponent 127 -> top 7 exponent bits 63 -> 0x3F
    assert list(hi) == [0x3F, 0xBF, 0x40, 0x3F, 0x80, 0x7F]


def _fp32_sweep():
    # every exponent x both signs x every value of each mantissa byte
    e = np.arange(256, dtype=np.uint32)
    s = np.arange(2, dtype=np.uint32)
    m = np.arange(256, dtype=np.uint32)
    parts = []
    for shift, mask in ((0, 0xFF), (8, 0xFF), (16, 0x7F)):
        mm = (m & mask) << shift
        grid = (s[:, None, None] << 31) | (e[None, :, None] << 23) | mm[None, None, :]
        parts.append(grid.ravel())
    return np.concatenate(parts)


def test_fp32_split_sweep(oracle_lib):
    o = oracle_lib
    u = _fp32_sweep()
    n = u.size
    exp, raw = o.split_fp32(u)
    b = u.view(np.uint8).reshape(-1, 4)
    sign = b[:, 3] >> 7
    e = ((b[:, 3] & 0x7F).astype(np.uint16) << 1 | (b[:, 2] >> 7)).astype(np.uint8)
    nsb = (n + 7) // 8
    assert raw.size == nsb + 3 * n
    assert np.array_equal(exp, e)
    assert np.array_equal(raw[:nsb], np.packbits(sign, bitorder="little"))
    assert np.array_equal(raw[nsb:nsb + n], b[:, 0])
    assert np.array_equal(raw[nsb + n:nsb + 2 * n], b[:, 1])
    assert np.array_equal(raw[nsb + 2 * n:], b[:, 2] & 0x7F)
    assert np.array_equal(o.merge_fp32(exp, raw), u)


@pytest.mark.parametrize("n", [1, 5, 8, 9, 65543])
def test_fp32_split_ragged(oracle_lib, n):
    o = oracle_lib
    g = np.random.default_rng(n)
    u = g.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)
    exp, raw = o.split_fp32(u)
    nsb = (n + 7) // 8
    sign = (u >> 31).astype(np.uint8)
    assert np.array_equal(raw[:nsb], np.packbits(sign, bitorder="little"))
    assert np.array_equal(o.merge_fp32(exp, raw), u)
