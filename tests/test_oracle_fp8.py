"""Pins of the oracle's FP8 layouts (CPU only).

The "PTWM" README ("How it works": bit reorder moves the exponent into the
high nibble of an 8-bit float; then a 2-plane nibble split).  The fields are
derived from the numeric value that torch's own float8 types assign to each
of the 256 byte patterns (sign from signbit, exponent and mantissa from
frexp), not from bit masks, so a wrong shift or mask in the oracle's split
fails them.
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")

ALL8 = np.arange(256, dtype=np.uint8)
SPEC = {"fp8e4m3": (torch.float8_e4m3fn, 4, 3, 7), "fp8e5m2": (torch.float8_e5m2, 5, 2, 15)}


def _fields(layout):
    """(sign, biased exponent, mantissa, is_nan) of all 256 patterns."""
    dt, ebits, mbits, bias = SPEC[layout]
    f = torch.from_numpy(ALL8.copy()).view(dt).to(torch.float64).numpy()
    sign = np.signbit(f).astype(np.uint32)
    nan = np.isnan(f)
    a = np.abs(np.where(nan, 0.0, f))
    fin = np.isfinite(a)
    tiny = 2.0 ** (1 - bias)
    m, e = np.frexp(np.where(fin & (a >= tiny), a, 1.0))
    exp = np.where(a >= tiny, e + bias - 1, 0)
    exp = np.where(~fin | nan, (1 << ebits) - 1, exp).astype(np.uint32)
    man = np.where(a >= tiny, (m * 2.0 - 1.0) * (1 << mbits), a / tiny * (1 << mbits))
    man = np.where(~fin, 0.0, man)
    assert np.all(man == np.round(man))
    return sign, exp, man.astype(np.uint32), nan


def _nibbles(raw, n):
    return np.stack([raw & 0xF, raw >> 4], axis=1).reshape(-1)[:n]


def test_e4m3_high_nibble_is_the_exponent():
    c, r = oracle.split_fp8("fp8e4m3", ALL8)
    s, e, m, nan = _fields("fp8e4m3")
    lo = _nibbles(r, 256)
    # e4m3fn has no infinity: its two NaN patterns carry mantissa 7
    m = np.where(nan, 7, m)
    assert np.array_equal(c, e)
    assert np.array_equal(lo >> 3, s)
    assert np.array_equal(lo & 7, m)


def test_e5m2_high_nibble_is_the_top_of_the_exponent():
    c, r = oracle.split_fp8("fp8e5m2", ALL8)
    s, e, m, nan = _fields("fp8e5m2")
    lo = _nibbles(r, 256)
    assert np.array_equal(c, e >> 1)
    assert np.array_equal(lo >> 3, e & 1)
    assert np.array_equal((lo >> 2) & 1, s)
    ok = ~nan
    assert np.array_equal((lo & 3)[ok], m[ok])
    assert np.all((lo & 3)[nan] != 0)     # NaN: non-zero mantissa (inf has zero)


@pytest.mark.parametrize("layout", ["fp8e4m3", "fp8e5m2"])
def test_fp8_split_is_a_bijection(layout):
    c, r = oracle.split_fp8(layout, ALL8)
    assert c.max() < 16
    pairs = c.astype(np.uint32) * 16 + _nibbles(r, 256)
    assert np.unique(pairs).size == 256
    assert np.array_equal(oracle.merge_fp8(layout, c, r), ALL8)


def test_fp8_nibble_packing_odd_count():
    v = np.array([0x38, 0xB9, 0x00, 0xFF, 0x47], np.uint8)   # 1.0, -1.125, 0, NaN, 288 (e4m3)
    c, r = oracle.split_fp8("fp8e4m3", v)
    assert r.size == 3 and (r[2] >> 4) == 0               # last high nibble unused, zero
    # element 0 (1.0 = 0 0111 000): exponent 7, sign 0, mantissa 0
    assert c[0] == 7 and (r[0] & 0xF) == 0
    # element 1 (-1.125 = 1 0111 001): exponent 7, sign 1, mantissa 1
    assert c[1] == 7 and (r[0] >> 4) == 0b1001
    assert np.array_equal(oracle.merge_fp8("fp8e4m3", c, r), v)


def _fp8_weights(layout, n, seed):
    dt, _, _, _ = SPEC[layout]
    x = torch.from_numpy(np.random.default_rng(seed).standard_normal(n).astype(np.float32))
    fmax = torch.finfo(dt).max
    return (x * (fmax / x.abs().max())).to(dt).view(torch.uint8).numpy()


@pytest.mark.parametrize("layout", ["fp8e4m3", "fp8e5m2"])
@pytest.mark.parametrize("opts", [0, oracle.OPT_TENSOR_TABLE | oracle.OPT_RAW_FALLBACK])
def test_fp8_round_trip_and_ratio(layout, opts):
    v = _fp8_weights(layout, 5 * 65536 + 777, 3)
    e = oracle.encode(v, layout, threads=4, opts=opts)
    assert e.raw.size == (v.size + 1) // 2
    y, err = oracle.decode(e, threads=4)
    assert err == 0 and np.array_equal(y, v)
    # the exponent nibble carries most of the redundancy: a Gaussian scaled to
    # the format's range compresses to the PTWM README's 0.70-0.85 bracket
    assert 0.70 <= e.total_bytes / v.size <= 0.88
    c, _ = oracle.split_fp8(layout, v)
    assert c.max() < 16 and np.unique(c).size > 4
