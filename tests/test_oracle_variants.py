"""Pins of the oracle's format variants (CPU only).

Layouts (the "PTWM" README, "How it works": bit reorder, then a 2-plane byte
split for 16-bit floats), tensor-wide tables and the raw-chunk fallback.  The
field checks derive sign, exponent and mantissa from float arithmetic
(numpy's frexp / signbit / isnan on the decoded value), not from bit masks, so
a wrong shift or mask in the oracle's split fails them.
"""
import numpy as np
import pytest

import oracle

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _fields_from_float(v16, kind):
    """(sign, biased exponent, mantissa, is_nan) of 16-bit patterns, computed
    from the numeric value: normal numbers from frexp, subnormals by scaling,
    infinities and NaNs by their class."""
    if kind == "bf16":
        with np.errstate(invalid="ignore"):
            f = (v16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ebits, mbits, bias = 8, 7, 127
    else:
        f = v16.view(np.float16).astype(np.float64)
        ebits, mbits, bias = 5, 10, 15
    emax = (1 << ebits) - 1
    sign = np.signbit(f).astype(np.uint32)
    nan = np.isnan(f)
    a = np.abs(np.where(nan, 0.0, f))
    fin = np.isfinite(a)
    tiny = 2.0 ** (1 - bias)                      # smallest normal
    m, e = np.frexp(np.where(fin & (a >= tiny), a, 1.0))
    exp = np.where(a >= tiny, e + bias - 1, 0)
    exp = np.where(~fin | nan, emax, exp).astype(np.uint32)
    frac_norm = (m * 2.0 - 1.0) * (1 << mbits)
    frac_sub = a / tiny * (1 << mbits)
    man = np.where(a >= tiny, frac_norm, frac_sub)
    man = np.where(~fin, 0.0, man)
    assert np.all(man == np.round(man))
    return sign, exp, man.astype(np.uint32), nan


def test_bf16_reorder_coded_byte_is_the_exponent():
    hi, lo = oracle.split_u16("bf16r", ALL16)
    s, e, m, nan = _fields_from_float(ALL16, "bf16")
    assert np.array_equal(hi, e)
    assert np.array_equal(lo >> 7, s)
    ok = ~nan
    assert np.array_equal((lo & 0x7F)[ok], m[ok])
    assert np.all((lo & 0x7F)[nan] != 0)          # NaN: non-zero mantissa


def test_bf16_plain_split_fields():
    hi, lo = oracle.split_u16("bf16", ALL16)
    s, e, m, nan = _fields_from_float(ALL16, "bf16")
    assert np.array_equal(hi >> 7, s)
    assert np.array_equal(hi & 0x7F, e >> 1)
    assert np.array_equal(lo >> 7, e & 1)
    assert np.array_equal((lo & 0x7F)[~nan], m[~nan])


def test_fp16_plain_split_fields():
    hi, lo = oracle.split_u16("fp16", ALL16)
    s, e, m, nan = _fields_from_float(ALL16, "fp16")
    assert np.array_equal(hi >> 7, s)
    assert np.array_equal((hi >> 2) & 0x1F, e)
    ok = ~nan
    assert np.array_equal((((hi & 3).astype(np.uint32) << 8) | lo)[ok], m[ok])


def test_fp16_reorder_fields():
    hi, lo = oracle.split_u16("fp16r", ALL16)
    s, e, m, nan = _fields_from_float(ALL16, "fp16")
    assert np.array_equal(hi >> 3, e)
    assert np.array_equal((hi >> 2) & 1, s)
    ok = ~nan
    assert np.array_equal((((hi & 3).astype(np.uint32) << 8) | lo)[ok], m[ok])
    assert np.all(((((hi & 3).astype(np.uint32) << 8) | lo)[nan]) != 0)


@pytest.mark.parametrize("layout", ["bf16", "bf16r", "fp16", "fp16r"])
def test_layouts_are_bijections(layout):
    hi, lo = oracle.split_u16(layout, ALL16)
    pairs = (hi.astype(np.uint32) << 8) | lo
    assert np.unique(pairs).size == 65536
    assert np.array_equal(oracle.merge_u16(layout, hi, lo), ALL16)


def test_bf16_split_matches_plain_bf16_entry_points():
    hi, lo = oracle.split_u16("bf16", ALL16)
    hi2, lo2 = oracle.split_bf16(ALL16)
    assert np.array_equal(hi, hi2) and np.array_equal(lo, lo2)


def _bf16_weights(n, seed=0, sigma=0.02):
    x = (np.random.default_rng(seed).standard_normal(n) * sigma).astype(np.float32)
    u = x.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _entropy(sym):
    c = np.bincount(sym, minlength=256).astype(np.float64)
    p = c[c > 0] / sym.size
    return float(-(p * np.log2(p)).sum())


def test_reorder_entropy_gain_is_the_chain_rule_difference():
    """H(sign, E>>1) - H(E) = H(sign | E>>1) - H(E0 | E>>1) exactly, on the
    empirical distribution; the reordered payload is smaller by about that."""
    v = _bf16_weights(1 << 20)
    hp, _ = oracle.split_u16("bf16", v)
    hr, _ = oracle.split_u16("bf16r", v)
    e_hi = (hr >> 1).astype(np.int64)
    sgn = (hp >> 7).astype(np.int64)
    e0 = (hr & 1).astype(np.int64)

    def cond(a, b):  # H(a | b)
        return _entropy_pairs(a, b) - _entropy_any(b)

    gain = cond(sgn, e_hi) - cond(e0, e_hi)
    assert abs((_entropy(hp) - _entropy(hr)) - gain) < 1e-9
    assert gain > 0.05
    ep = oracle.encode(v, "bf16", threads=4)
    er = oracle.encode(v, "bf16r", threads=4)
    bits = 8.0 * (er.payload.size - ep.payload.size) / v.size
    assert abs(bits + gain) < 0.01


def _entropy_any(a):
    _, c = np.unique(a, return_counts=True)
    p = c / a.size
    return float(-(p * np.log2(p)).sum())


def _entropy_pairs(a, b):
    return _entropy_any(a * 1024 + b)


# ------------------------------------------------------------ normalise64

def test_normalize64_hand_example_three_equal_symbols():
    # q = 4096 // 3 = 1365 each, remainders equal, D = 1 goes to symbol 0
    c = np.zeros(256, np.uint64)
    c[[3, 7, 200]] = 1 << 38
    f = oracle.normalize64(c)
    want = np.zeros(256, np.uint16)
    want[[3, 7, 200]] = [1366, 1365, 1365]
    assert np.array_equal(f, want)


def test_normalize64_forced_symbols_taken_from_the_largest():
    # one symbol with 2^40 - 255, 255 symbols with count 1: those are forced
    # to 1; the big one's q = 4095, so D = -254 comes off it: 3841
    c = np.ones(256, np.uint64)
    c[0] = (1 << 40) - 255
    f = oracle.normalize64(c)
    assert f[0] == 3841 and np.all(f[1:] == 1)


def test_normalize64_exact_scaling_returns_the_table():
    rng = np.random.default_rng(5)
    for _ in range(20):
        k = int(rng.integers(1, 200))
        syms = rng.choice(256, k, replace=False)
        cuts = np.sort(rng.choice(np.arange(1, 4096), k - 1, replace=False))
        parts = np.diff(np.concatenate([[0], cuts, [4096]]))
        f = np.zeros(256, np.uint16)
        f[syms] = parts
        c = f.astype(np.uint64) << np.uint64(28)
        assert np.array_equal(oracle.normalize64(c), f)


def test_normalize64_agrees_with_chunk_normalize():
    rng = np.random.default_rng(6)
    for _ in range(200):
        k = int(rng.integers(1, 257))
        c = np.zeros(256, np.uint32)
        c[rng.choice(256, k, replace=False)] = rng.integers(1, 3000, k)
        assert np.array_equal(oracle.normalize64(c.astype(np.uint64)), oracle.normalize(c))


# ----------------------------------------------------------- tensor table

def test_tensor_table_one_chunk_equals_chunk_table():
    v = _bf16_weights(50000, seed=1)
    a = oracle.encode(v, "bf16")
    b = oracle.encode(v, "bf16", opts=oracle.OPT_TENSOR_TABLE)
    assert np.array_equal(a.tables, b.tables)
    assert np.array_equal(a.seek, b.seek) and np.array_equal(a.payload, b.payload)


def test_tensor_table_of_repeated_chunk_is_its_table():
    one = _bf16_weights(65536, seed=2)
    v = np.tile(one, 5)
    a = oracle.encode(one, "bf16")
    b = oracle.encode(v, "bf16", opts=oracle.OPT_TENSOR_TABLE)
    assert b.tables.shape == (1, 256)
    assert np.array_equal(b.tables[0], a.tables[0])
    size = int(a.seek[1])
    assert np.array_equal(np.diff(b.seek.astype(np.int64)), [size] * 5)
    for k in range(5):
        assert np.array_equal(b.payload[k * size:(k + 1) * size], a.payload)


@pytest.mark.parametrize("layout", ["bf16", "bf16r", "fp16", "fp32"])
def test_tensor_table_round_trip_and_saving(layout):
    n = 7 * 65536 + 1234
    if layout == "fp32":
        x = (np.random.default_rng(3).standard_normal(n) * 0.02).astype(np.float32).view(np.uint32)
    elif layout == "fp16":
        x = (np.random.default_rng(3).standard_normal(n) * 0.02).astype(np.float16).view(np.uint16)
    else:
        x = _bf16_weights(n, seed=3)
    a = oracle.encode(x, layout, threads=4)
    b = oracle.encode(x, layout, threads=4, opts=oracle.OPT_TENSOR_TABLE)
    y, err = oracle.decode(b, threads=4)
    assert err == 0 and np.array_equal(y, x)
    assert b.tables.size == 256 and a.tables.shape[0] == 8
    saved = a.total_bytes - b.total_bytes
    assert 0 < saved < 512 * 7          # tables saved, minus a small coding cost


def test_tensor_table_is_the_whole_plane_histogram_normalised():
    # chunks with different supports: the table must cover all of them
    parts = [_bf16_weights(65536, seed=10, sigma=s) for s in (0.001, 0.02, 0.5)]
    v = np.concatenate(parts + [_bf16_weights(999, seed=11, sigma=3.0)])
    e = oracle.encode(v, "bf16", threads=2, opts=oracle.OPT_TENSOR_TABLE)
    hi, _ = oracle.split_u16("bf16", v)
    counts = np.bincount(hi, minlength=256).astype(np.uint64)
    assert np.array_equal(e.tables[0], oracle.normalize64(counts, v.size))
    assert np.array_equal((e.tables[0] > 0), counts > 0)
    y, err = oracle.decode(e, threads=2)
    assert err == 0 and np.array_equal(y, v)


def test_tensor_table_empty_tensor_has_zero_table():
    e = oracle.encode(np.zeros(0, np.uint16), "bf16", opts=oracle.OPT_TENSOR_TABLE)
    assert e.tables.shape == (1, 256) and not e.tables.any()


# ------------------------------------------------------------ raw fallback

def _uniform_chunk(seed=4):
    s = np.repeat(np.arange(256, dtype=np.uint16), 256)
    np.random.default_rng(seed).shuffle(s)
    return s


def test_raw_fallback_stores_a_uniform_chunk_as_its_symbols():
    hi = _uniform_chunk()
    lo = np.random.default_rng(1).integers(0, 256, 65536).astype(np.uint16)
    v = (hi << 8) | lo
    plain = oracle.encode(v, "bf16")
    assert int(plain.seek[1]) > 65536                 # coding expands it
    e = oracle.encode(v, "bf16", opts=oracle.OPT_RAW_FALLBACK)
    assert int(e.seek[1]) == 65536
    assert np.array_equal(e.payload, hi.astype(np.uint8))
    assert np.array_equal(e.tables, plain.tables)     # the table is still written
    y, err = oracle.decode(e)
    assert err == 0 and np.array_equal(y, v)


def test_raw_fallback_keeps_skewed_chunks_coded():
    v = _bf16_weights(3 * 65536 + 100, seed=7)
    a = oracle.encode(v, "bf16")
    b = oracle.encode(v, "bf16", opts=oracle.OPT_RAW_FALLBACK)
    assert np.array_equal(a.seek[:4], b.seek[:4])
    assert np.array_equal(a.payload[: int(a.seek[3])], b.payload[: int(b.seek[3])])


def test_raw_fallback_short_tail_and_padding():
    v = _bf16_weights(65536 + 5, seed=8)
    e = oracle.encode(v, "bf16", opts=oracle.OPT_RAW_FALLBACK)
    # a 5-symbol chunk codes to >= 128 bytes, so it is stored raw in 8 bytes
    assert int(e.seek[2] - e.seek[1]) == 8
    tail = e.payload[int(e.seek[1]):]
    assert np.array_equal(tail[:5], (v[65536:] >> 8).astype(np.uint8)) and not tail[5:].any()
    lay = oracle.query_layout("bf16", v.size, oracle.OPT_RAW_FALLBACK)
    assert lay.payload_capacity == 65536 + 8
    y, err = oracle.decode(e)
    assert err == 0 and np.array_equal(y, v)
    bad = oracle.Encoded(e.dtype, e.n, e.raw, e.tables, e.seek, e.payload.copy(), e.opts)
    bad.payload[-1] = 1
    _, err = oracle.decode(bad, strict=False)
    assert err & oracle.EF_BAD_TAIL


def test_raw_fallback_with_tensor_table_fp32():
    n = 3 * 65536
    rng = np.random.default_rng(9)
    u = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)   # uniform exponents
    u[65536:] = (rng.standard_normal(2 * 65536) * 0.02).astype(np.float32).view(np.uint32)
    opts = oracle.OPT_RAW_FALLBACK | oracle.OPT_TENSOR_TABLE
    e = oracle.encode(u, "fp32", threads=3, opts=opts)
    y, err = oracle.decode(e, threads=3)
    assert err == 0 and np.array_equal(y, u)


def test_batch_with_options():
    xs = [_bf16_weights(n, seed=i) for i, n in enumerate([70000, 0, 65536, 3])]
    opts = oracle.OPT_TENSOR_TABLE | oracle.OPT_RAW_FALLBACK
    e = oracle.encode_batch(xs, "bf16r", threads=2, opts=opts)
    assert e.tables.shape == (4, 256)
    outs, err = oracle.decode_batch(e, threads=2)
    assert err == 0 and all(np.array_equal(a, b) for a, b in zip(outs, xs))
    # every tensor's slice equals its own single-tensor encoding
    for i, x in enumerate(xs):
        one = oracle.encode(x, "bf16r", opts=opts)
        assert np.array_equal(e.tables[i], one.tables[0])


# ----------------------------------------------------------------- CRC-32

def test_crc32_check_value():
    # the CRC-32/ISO-HDLC catalogue check value: CRC of the ASCII digits 1..9
    assert oracle.crc32(b"123456789") == 0xCBF43926
    assert oracle.crc32(b"") == 0


def test_crc32_matches_zlib():
    import zlib
    g = np.random.default_rng(41)
    for n in (1, 3, 4, 63, 64, 65, 1000, 21847, 131200):
        a = g.integers(0, 256, n).astype(np.uint8)
        assert oracle.crc32(a) == zlib.crc32(a.tobytes())


def test_chunk_crc_of_an_encoding():
    import zlib
    v = _bf16_weights(3 * 65536 + 5, seed=42)
    e = oracle.encode(v, "bf16", opts=oracle.OPT_CRC32)
    plain = oracle.encode(v, "bf16")
    assert np.array_equal(e.payload, plain.payload) and np.array_equal(e.seek, plain.seek)
    crc = oracle.chunk_crc(e.seek, e.payload)
    for k in range(4):
        assert crc[k] == zlib.crc32(e.payload[int(e.seek[k]):int(e.seek[k + 1])].tobytes())
