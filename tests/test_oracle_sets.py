"""Oracle on the FP32 path and on batches of tensors.

FP32 follows the SMEF README's pass 3 (sign / exponent / mantissa byte
streams, only the exponent coded); batches follow the PTWM README's
multi-tensor container idea: every tensor is coded on its own and the parts
are laid end to end.
"""
import numpy as np
import pytest

from lossless_weight_compression_bf16_amd import synthetic as S


def test_fp32_config_round_trip_and_ratio(oracle_lib):
    w = S.workload("fp32-768x2304")
    u = S.tensor_bits(w, 0)
    e = oracle_lib.encode(u, "fp32")
    y, err = oracle_lib.decode(e)
    assert err == 0 and np.array_equal(y, u)
    ex = ((u >> 23) & 0xFF).astype(np.uint8)
    c = np.bincount(ex, minlength=256)
    p = c[c > 0] / c.sum()
    H = float(-(p * np.log2(p)).sum())
    assert 2.3 <= H <= 2.8
    ratio = e.total_bytes / (4 * u.size)
    # sign bit + 23 mantissa bits raw (3.125 B/elem incl. the top m2 bit), exponent ~H bits
    expect = (1 + 24 + H + 0.079) / 32
    assert abs(ratio - expect) < 0.01


def test_fp32_is_the_bf16_config_before_rounding():
    a = S.tensor_bits(S.workload("fp32-768x2304"), 0)
    b = S.tensor_bits(S.workload("bf16-768x2304"), 0)
    assert np.array_equal(S.f32_to_bf16_bits(a.view(np.float32)), b)


def test_fp32_special_patterns(oracle_lib):
    pats = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00001, 0x00000001,
                     0x807FFFFF, 0x3F800000], np.uint32)
    x = np.tile(pats, 9000)
    e = oracle_lib.encode(x, "fp32")
    y, err = oracle_lib.decode(e)
    assert err == 0 and np.array_equal(x, y)


def test_batch_is_concatenation(oracle_lib):
    g = np.random.default_rng(2)
    xs = [S.f32_to_bf16_bits((g.standard_normal(n) * 0.02).astype(np.float32))
          for n in (65536 * 2 + 5, 1, 0, 70000, 300)]
    b = oracle_lib.encode_batch(xs, "bf16")
    cb, rb, tot = oracle_lib.plan_batch("bf16", [x.size for x in xs])
    base = 0
    for i, x in enumerate(xs):
        e = oracle_lib.encode(x, "bf16")
        c = e.tables.shape[0]
        k0 = int(cb[i])
        assert np.array_equal(b.tables[k0:k0 + c], e.tables)
        assert np.array_equal(b.seek[k0:k0 + c + 1] - b.seek[k0], e.seek)
        assert int(b.seek[k0]) == base
        assert np.array_equal(b.payload[base: base + e.payload.size], e.payload)
        assert np.array_equal(b.raw[int(rb[i]): int(rb[i]) + x.size], e.raw)
        assert int(rb[i]) % 256 == 0
        base += e.payload.size
    outs, err = oracle_lib.decode_batch(b)
    assert err == 0
    for x, y in zip(xs, outs):
        assert np.array_equal(x, y)


def test_empty_tensor(oracle_lib):
    e = oracle_lib.encode(np.zeros(0, np.uint16), "bf16")
    assert list(e.seek) == [0] and e.payload.size == 0 and e.raw.size == 0
    y, err = oracle_lib.decode(e)
    assert y.size == 0 and err == 0


@pytest.mark.parametrize("threads", [1, 3, 8])
def test_threads_do_not_change_bytes(oracle_lib, threads):
    g = np.random.default_rng(8)
    x = S.f32_to_bf16_bits((g.standard_normal(65536 * 7 + 3) * 0.02).astype(np.float32))
    ref = oracle_lib.encode(x, "bf16", threads=1)
    e = oracle_lib.encode(x, "bf16", threads=threads)
    assert np.array_equal(e.payload, ref.payload) and np.array_equal(e.seek, ref.seek)
    y, err = oracle_lib.decode(e, threads=threads)
    assert err == 0 and np.array_equal(x, y)
