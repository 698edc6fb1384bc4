"""GPU path against the oracle, element by element and byte by byte.

Every integer result must be identical: frequency tables, seek table,
payload bytes, raw planes and decoded bit patterns (the Split12 README's
bit-for-bit bar; the format is integer-only, so there is no tolerance).
All calls go through the C ABI via the ctypes binding.
"""
import json
import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import lossless_weight_compression_bf16_amd as wc  # noqa: E402
from lossless_weight_compression_bf16_amd import codec, synthetic as S  # noqa: E402


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    wc.lib()  # a missing library is an error here, not a skip
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _weights(n, seed, sigma=0.02):
    g = np.random.default_rng(seed)
    return S.f32_to_bf16_bits((g.standard_normal(n) * sigma).astype(np.float32))


def _to_dev(a, dev, dtype):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16 if dtype == "bf16" else np.int32)).to(dev)


def _compare(e, o, what):
    h = e.to_host()
    assert np.array_equal(h["tables"].reshape(-1), o.tables.reshape(-1)), f"{what}: tables"
    assert np.array_equal(h["seek"], o.seek), f"{what}: seek"
    assert np.array_equal(h["payload"], o.payload), f"{what}: payload"
    assert np.array_equal(h["raw"], o.raw), f"{what}: raw planes"


def _upload(o, dev):
    """An oracle encoding as a device-side Encoded (for GPU decode of oracle bytes)."""
    def t(a, dt):
        a = np.ascontiguousarray(a)
        if a.size == 0:
            a = np.zeros(16 // np.dtype(dt).itemsize, dt)
        return torch.from_numpy(a.view(dt)).to(dev)
    shape = (o.n,)
    tdt = torch.bfloat16 if o.dtype == "bf16" else torch.float32
    raw = t(o.raw, np.uint8)[: o.raw.size]
    tables = t(o.tables.reshape(-1), np.int16)[: o.tables.size]
    seek = t(o.seek, np.int64)
    payload = t(o.payload, np.uint8)[: o.payload.size]
    return codec.Encoded(o.dtype, o.n, shape, tdt, raw, tables, seek, payload)


def _round_trip(x, dtype, dev, oracle_lib, what):
    _say(f"[parity] {what}: n={x.size} dtype={dtype}")
    xt = _to_dev(x, dev, dtype)
    xt = xt.view(torch.bfloat16) if dtype == "bf16" else xt.view(torch.float32)
    e = codec.encode(xt)
    o = oracle_lib.encode(x, dtype, threads=8)
    _compare(e, o, what)
    y = codec.decode(e)
    assert torch.equal(y.view(torch.int16 if dtype == "bf16" else torch.int32).cpu(),
                       xt.view(torch.int16 if dtype == "bf16" else torch.int32).cpu()), f"{what}: decode"
    z = codec.decode(_upload(o, dev))
    assert torch.equal(z.view(y.dtype).view(torch.int16 if dtype == "bf16" else torch.int32).cpu(),
                       xt.view(torch.int16 if dtype == "bf16" else torch.int32).cpu()), f"{what}: oracle bytes"
    return e, o


SIZES = [1, 2, 31, 32, 33, 1000, 65535, 65536, 65537, 2 * 65536, 3 * 65536, 3 * 65536 + 12345]


@pytest.mark.parametrize("n", SIZES)
def test_bf16_sizes(dev, oracle_lib, n):
    _round_trip(_weights(n, n), "bf16", dev, oracle_lib, f"bf16 n={n}")


@pytest.mark.parametrize("n", [1, 9, 65536, 65537, 3 * 65536 + 7])
def test_fp32_sizes(dev, oracle_lib, n):
    g = np.random.default_rng(n)
    x = (g.standard_normal(n) * 0.02).astype(np.float32).view(np.uint32)
    _round_trip(x, "fp32", dev, oracle_lib, f"fp32 n={n}")


def test_every_bf16_pattern(dev, oracle_lib):
    v = np.arange(65536, dtype=np.uint16)
    g = np.random.default_rng(1)
    x = np.concatenate([g.permutation(v), v, g.permutation(v)[:40000]])
    _round_trip(x, "bf16", dev, oracle_lib, "all bf16 patterns")


def test_fp32_special_patterns(dev, oracle_lib):
    pats = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00001, 0x00000001, 0x807FFFFF,
                     0x3F800000], np.uint32)
    g = np.random.default_rng(2)
    x = g.permutation(np.tile(pats, 20000))
    _round_trip(x, "fp32", dev, oracle_lib, "fp32 specials")


def test_table_edge_cases(dev, oracle_lib):
    """Single symbol (f = 4096), two symbols, uniform 256 (f = 16), many
    forced rare symbols (negative shortfall), ties in remainders."""
    g = np.random.default_rng(3)
    parts = [
        np.full(65536, 0x3C11, np.uint16),
        np.where(g.random(65536) < 0.5, 0x3C00, 0xBC00).astype(np.uint16) | g.integers(0, 256, 65536).astype(np.uint16),
        g.permutation(np.arange(65536, dtype=np.uint16)),
        np.concatenate([np.full(65536 - 255, 0x3C00, np.uint16),
                        (np.arange(256, dtype=np.uint16)[np.arange(256) != 0x3C] << 8)]),
        S.f32_to_bf16_bits((g.standard_t(1.2, 65536) * 0.01).astype(np.float32)),
        np.full(12345, 0xFF80, np.uint16),
    ]
    x = np.concatenate([g.permutation(p) if i in (3, 4) else p for i, p in enumerate(parts)])
    _round_trip(x, "bf16", dev, oracle_lib, "table edge cases")


def test_high_entropy_chunks_next_to_weights(dev, oracle_lib):
    """Chunks whose coded byte is uniform over 256 values need about 128
    stream words per 8-step group, more than the decoder refills per group:
    their first speculative pass overruns the landed words and the chunk is
    decoded again from its start.  Alternating them with weight chunks puts
    one of each in every two-chunk wavefront (and an odd count leaves a
    shadow half), so a redo next to a half that did not need one is covered."""
    g = np.random.default_rng(11)
    parts = []
    for k in range(7):
        if k % 2:
            parts.append(g.integers(0, 65536, 65536, dtype=np.uint64).astype(np.uint16))
        else:
            parts.append(_weights(65536, 100 + k))
    parts.append(g.integers(0, 65536, 4321, dtype=np.uint64).astype(np.uint16))
    _round_trip(np.concatenate(parts), "bf16", dev, oracle_lib, "high-entropy chunks")


def test_two_chunk_wavefronts_with_redo(dev, oracle_lib):
    """Above eight chunks per compute unit (2048 on a 256-CU device) the
    decoder runs two chunks per wavefront with the small word ring.  2401
    chunks (an odd count, so the last wavefront has a shadow half), weights
    throughout except every 37th chunk and the last three, which are
    uniform over all 65536 patterns and overrun the refill rate."""
    nchunks = 2401
    g = np.random.default_rng(12)
    x = _weights(65536 * (nchunks - 1) + 4321, 13)
    hot = [k for k in range(nchunks) if k % 37 == 5] + [nchunks - 3, nchunks - 2, nchunks - 1]
    for k in hot:
        a, b = 65536 * k, min(65536 * (k + 1), x.size)
        x[a:b] = g.integers(0, 65536, b - a, dtype=np.uint64).astype(np.uint16)
    _round_trip(x, "bf16", dev, oracle_lib, "two-chunk wavefronts")


def test_golden_streams_on_gpu(dev):
    path = os.path.join(os.path.dirname(__file__), "golden", "chunk_streams.json")
    cases = json.load(open(path))["cases"]
    sys.path.insert(0, os.path.dirname(__file__))
    from test_oracle_rans import _input, _states
    for case in cases:
        x = _input(case)
        dtype = case["dtype"]
        xt = _to_dev(x, dev, dtype)
        e = codec.encode(xt.view(torch.bfloat16 if dtype == "bf16" else torch.float32))
        h = e.to_host()
        assert list(h["payload"][:128].view("<u4")) == _states(case), case["name"]
        words = [int(w, 16) for w in case["words_u16"]]
        assert list(h["payload"][128:].view("<u2")[: len(words)]) == words, case["name"]
        assert h["payload"].size == case["payload_bytes"], case["name"]


def test_bf16_768x2304_full(dev, oracle_lib):
    w = S.workload("bf16-768x2304")
    _round_trip(S.tensor_bits(w, 0), "bf16", dev, oracle_lib, w.name)


def test_fp32_768x2304_full(dev, oracle_lib):
    w = S.workload("fp32-768x2304")
    _round_trip(S.tensor_bits(w, 0), "fp32", dev, oracle_lib, w.name)


def _batch_parity(xs, dtype, dev, oracle_lib, what):
    _say(f"[parity] batch {what}: {len(xs)} tensors, {sum(x.size for x in xs)} elements")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ts = [_to_dev(x, dev, dtype).view(tdt) for x in xs]
    e = codec.encode_batch(ts)
    o = oracle_lib.encode_batch(xs, dtype, threads=16)
    assert np.array_equal(e.tables.cpu().numpy().view("<u2").reshape(-1), o.tables.reshape(-1)), what
    assert np.array_equal(e.seek.cpu().numpy().view("<u8"), o.seek), what
    assert np.array_equal(e.payload.cpu().numpy(), o.payload), what
    assert np.array_equal(e.raw.cpu().numpy(), o.raw), what
    ys = codec.decode_batch(e)
    ity = torch.int16 if dtype == "bf16" else torch.int32
    for t, y in zip(ts, ys):
        assert torch.equal(t.view(ity), y.view(ity)), what
    return e, o


def test_batch_edges(dev, oracle_lib):
    xs = [_weights(n, i) for i, n in enumerate([65536 * 2 + 5, 1, 0, 70000, 300, 65536, 33])]
    _batch_parity(xs, "bf16", dev, oracle_lib, "edges")


def test_gpt2_small_set_full(dev, oracle_lib):
    w = S.workload("gpt2-small-bf16")
    xs = S.set_bits(w)
    e, o = _batch_parity(xs, "bf16", dev, oracle_lib, w.name)
    _say(f"[parity] {w.name}: ratio {e.ratio:.4f}")


def _mixed_chunks(g, nchunks, tail):
    """Chunks of varied entropy, one kind each: weights of random scale,
    heavy-tailed values, uniform 16-bit patterns, a constant, two values, and
    values confined to a few exponents; then a ragged tail of weights."""
    parts = []
    for _ in range(nchunks):
        kind = int(g.integers(0, 6))
        if kind == 0:
            c = _weights(65536, int(g.integers(1 << 30)), float(g.uniform(0.001, 0.2)))
        elif kind == 1:
            c = S.f32_to_bf16_bits((g.standard_t(3, 65536) * 0.015).astype(np.float32))
        elif kind == 2:
            c = g.integers(0, 65536, 65536, dtype=np.uint64).astype(np.uint16)
        elif kind == 3:
            c = np.full(65536, int(g.integers(0, 65536)), np.uint16)
        elif kind == 4:
            c = np.where(g.random(65536) < 0.3, 0x3C00, 0xBC80).astype(np.uint16)
        else:
            c = ((g.integers(0x78, 0x7C, 65536) << 8) | g.integers(0, 256, 65536)).astype(np.uint16)
        parts.append(c)
    parts.append(_weights(tail, int(g.integers(1 << 30))))
    return np.concatenate(parts)


@pytest.mark.parametrize("seed", range(8))
def test_mixed_entropy_chunks(dev, oracle_lib, seed):
    """Random mixes of chunk kinds and counts (1 to 12 chunks plus a ragged
    tail): the one-chunk-per-wavefront decoder with either refill width
    (chosen by the mix's average bits per symbol), redo passes on the
    near-uniform chunks, partial last groups and ring wrap-around, all
    against the oracle's bytes."""
    g = np.random.default_rng(500 + seed)
    x = _mixed_chunks(g, int(g.integers(1, 13)), int(g.integers(0, 65536)))
    _round_trip(x, "bf16", dev, oracle_lib, f"mixed chunks, seed {seed}")


def test_deterministic(dev):
    x = _to_dev(_weights(5 * 65536 + 3, 9), dev, "bf16").view(torch.bfloat16)
    a = codec.encode(x).to_host()
    b = codec.encode(x).to_host()
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_capacity_overflow_is_reported(dev):
    from lossless_weight_compression_bf16_amd import _binding as B
    x = _to_dev(_weights(3 * 65536, 4), dev, "bf16")
    lay = B.wc_query_layout("bf16", x.numel())
    raw = torch.empty(lay.raw_bytes, dtype=torch.uint8, device=dev)
    tables = torch.empty(lay.num_chunks * 256, dtype=torch.int16, device=dev)
    seek = torch.empty(lay.num_chunks + 1, dtype=torch.int64, device=dev)
    payload = torch.zeros(4096, dtype=torch.uint8, device=dev)
    scratch = torch.empty(lay.scratch_bytes, dtype=torch.uint8, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    bufs = B.make_buffers(raw, tables, seek, payload, payload.numel())
    B.wc_encode("bf16", x, x.numel(), bufs, scratch, scratch.numel(), err)
    torch.cuda.synchronize()
    assert int(err.item()) & B.EF_CAPACITY


def test_corrupt_streams_are_flagged(dev, oracle_lib):
    """Flipped payload bytes, bad tables and bad seek entries give error bits
    or a different tensor; the decoder keeps every access in bounds."""
    x = _weights(3 * 65536 + 100, 5)
    o = oracle_lib.encode(x, "bf16")
    g = np.random.default_rng(6)
    xt = torch.from_numpy(x.view(np.int16))
    detected = 0
    trials = 40
    for trial in range(trials):
        import copy
        d = copy.deepcopy(o)
        kind = trial % 4
        if kind == 0:
            i = int(g.integers(0, d.payload.size))
            d.payload[i] ^= np.uint8(1 << int(g.integers(0, 8)))
        elif kind == 1:
            d.payload = d.payload[: int(g.integers(0, d.payload.size))]
        elif kind == 2:
            k = int(g.integers(0, d.tables.shape[0]))
            s = int(g.integers(0, 256))
            d.tables[k, s] = np.uint16(int(d.tables[k, s]) + int(g.integers(1, 5)))
        else:
            k = int(g.integers(1, d.seek.size))
            d.seek[k] = np.uint64(int(d.seek[k]) + 4 * int(g.integers(1, 1000)))
        e = _upload(d, dev)
        y = codec.decode(e, check=False)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        from lossless_weight_compression_bf16_amd import _binding as B
        B.wc_decode("bf16", e.buffers(), e.n, y.view(torch.int16), err)
        bits = int(err.item())
        ok = torch.equal(y.view(torch.int16).cpu(), xt)
        if bits or not ok:
            detected += 1
        # the oracle flags the same streams
        _, obits = oracle_lib.decode(d, strict=False)
        assert (bits != 0) == (obits != 0), (trial, bits, obits)
    assert detected >= trials - 4


def test_corrupt_streams_two_chunk_wavefronts(dev, oracle_lib):
    """The corruption kinds above on a tensor of 2101 chunks, decoded two
    chunks per wavefront: error bits agree with the oracle and every access
    stays in bounds."""
    import copy
    from lossless_weight_compression_bf16_amd import _binding as B
    x = _weights(65536 * 2100 + 777, 14)
    o = oracle_lib.encode(x, "bf16", threads=8)
    g = np.random.default_rng(15)
    for trial in range(8):
        d = copy.deepcopy(o)
        kind = trial % 4
        k = int(g.integers(0, d.tables.shape[0]))
        if kind == 0:
            i = int(g.integers(int(d.seek[k]), int(d.seek[k + 1])))
            d.payload[i] ^= np.uint8(1 << int(g.integers(0, 8)))
        elif kind == 1:
            d.payload = d.payload[: int(d.seek[k]) + int(g.integers(0, 200))]
        elif kind == 2:
            d.tables[k, int(g.integers(0, 256))] += np.uint16(int(g.integers(1, 5)))
        else:
            d.seek[k + 1] = np.uint64(int(d.seek[k + 1]) + 4 * int(g.integers(1, 1000)))
        _say(f"[parity] corrupt two-chunk trial {trial} kind {kind} chunk {k}")
        e = _upload(d, dev)
        y = torch.empty(x.size, dtype=torch.int16, device=dev)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        B.wc_decode("bf16", e.buffers(), e.n, y, err)
        bits = int(err.item())
        oy, obits = oracle_lib.decode(d, threads=8, strict=False)
        assert (bits != 0) == (obits != 0), (trial, bits, obits)
        if bits == 0:
            # an undetected change decodes to the same bytes on both sides
            assert np.array_equal(y.cpu().numpy().view(np.uint16), oy), trial



@pytest.mark.parametrize("n_chunks", [3, 2101])
def test_stored_state_below_L_is_flagged(dev, oracle_lib, n_chunks):
    """A chunk whose stored states include one below L = 2^16 is no encoding:
    both decoder forms (one chunk per wavefront for 3 chunks, two for 2101)
    report BAD_FINAL_STATE, the same bits as the oracle, and decode the other
    chunks bit for bit."""
    import copy
    from lossless_weight_compression_bf16_amd import _binding as B
    x = _weights(65536 * (n_chunks - 1) + 999, 21)
    o = oracle_lib.encode(x, "bf16", threads=8)
    g = np.random.default_rng(22)
    for trial, v in enumerate((0, 1, 65535)):
        d = copy.deepcopy(o)
        k = int(g.integers(0, n_chunks))
        lane = int(g.integers(0, 32))
        at = int(d.seek[k]) + 4 * lane
        d.payload[at:at + 4] = np.frombuffer(np.uint32(v).tobytes(), np.uint8)
        _say(f"[parity] stored state {v} in chunk {k} lane {lane} of {n_chunks}")
        e = _upload(d, dev)
        y = torch.empty(x.size, dtype=torch.int16, device=dev)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        B.wc_decode("bf16", e.buffers(), e.n, y, err)
        bits = int(err.item())
        oy, obits = oracle_lib.decode(d, threads=8, strict=False)
        assert bits == obits == oracle_lib.EF_BAD_FINAL_STATE, (trial, bits, obits)
        keep = np.ones(x.size, bool)
        keep[65536 * k:65536 * (k + 1)] = False
        assert np.array_equal(y.cpu().numpy().view(np.uint16)[keep], x[keep]), trial


def test_decoder_variant_follows_the_streams_device(dev):
    """The decoder is picked from the CU count of the device the stream
    belongs to: one chunk per wavefront while every chunk fits at once (8
    wavefronts per CU with one-dword refills, 7 with two-dword ones), two per
    wavefront above; the same answer on the null stream and on a stream of
    that device."""
    from lossless_weight_compression_bf16_amd import _binding as B
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    side = torch.cuda.Stream(device=dev)
    for stream in (None, side):
        for per_cu, bytes_per_chunk, dwords in ((8, 22000, 1), (7, 60000, 2)):
            c = per_cu * cus
            for chunks, one in ((c, True), (c + 1, False)):
                got = B.wc_decode_variant("bf16", chunks, chunks * 65536, chunks * bytes_per_chunk, stream)
                assert got == (one, dwords), (stream, per_cu, chunks, got)
