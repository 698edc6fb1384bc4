"""Pins of the oracle's chunked rANS coder.

No page prints a worked example or fixes rANS parameters, so the oracle is
pinned by (a) hand-derived streams (tests/golden/chunk_streams.json) that fix
the state arithmetic, the lane mapping and the word order, (b) closed-form
special streams, (c) a provable size bound against the entropy of the chunk
under its own 12-bit table, and (d) exact round trips, including every BF16
bit pattern.  The round-trip bar is the weight-compression (Split12) README's
bit-for-bit criterion.
"""
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "chunk_streams.json")
L = 65536


def _golden():
    with open(GOLDEN) as fh:
        return {c["name"]: c for c in json.load(fh)["cases"]}


def _input(case):
    spec = case.get("input_u16") or case.get("input_u32")
    if "fill" in spec:
        return np.full(spec["count"], int(spec["fill"], 16), np.uint16)
    if "values" in spec:
        dt = np.uint16 if "input_u16" in case else np.uint32
        return np.array([int(v, 16) for v in spec["values"]], dt)
    hi = np.full(spec["count"], int(spec["other_hi"], 16), np.uint16)
    for t in range(8):
        hi[32 * t] = int(spec["lane0_hi"][t], 16)
        hi[32 * t + 1] = int(spec["lane1_hi"][t], 16)
    return (hi << 8) | (np.arange(spec["count"]) & 0xFF).astype(np.uint16)


def _states(case):
    st = case["states_u32"]
    if "all" in st:
        return [st["all"]] * 32
    return [st.get(str(l), st.get("rest")) for l in range(32)]


@pytest.mark.parametrize("name", list(_golden()))
def test_golden_streams(oracle_lib, name):
    case = _golden()[name]
    x = _input(case)
    e = oracle_lib.encode(x, case["dtype"])
    exp_table = np.zeros(256, np.uint16)
    for k, v in case["tables"].items():
        exp_table[int(k, 16)] = v
    assert np.array_equal(e.tables[0], exp_table)
    p = e.payload
    assert p.size == case["payload_bytes"]
    assert list(e.seek) == [0, case["payload_bytes"]]
    assert list(p[:128].view("<u4")) == _states(case)
    words = [int(w, 16) for w in case["words_u16"]]
    body = p[128:].view("<u2")
    assert list(body[: len(words)]) == words
    assert np.all(body[len(words):] == 0)
    if case["dtype"] == "bf16":
        assert np.array_equal(e.raw, (x & 0xFF).astype(np.uint8))
    else:
        planes = case["raw_planes"]
        ref = np.array([int(v, 16) for k in ("sign", "m0", "m1", "m2") for v in planes[k]], np.uint8)
        assert np.array_equal(e.raw, ref)
    y, err = oracle_lib.decode(e)
    assert err == 0 and np.array_equal(y, x)


def _hq_bits(sym, f):
    c = np.bincount(sym, minlength=256)
    nz = c > 0
    return float((c[nz] * np.log2(4096.0 / f[nz].astype(np.float64))).sum())


def _size_bound(n, hq):
    # 32 states + at most one pad word + what the proof allows for the words
    return 128 + 2 + (hq + n * math.log2(17.0 / 16.0)) / 8.0


def _weights_like(g, n, sigma=0.02):
    v = (g.standard_normal(n) * sigma).astype(np.float32)
    u = v.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_all_same_symbol(oracle_lib):
    for n in (1, 31, 32, 33, 65536):
        sym = np.full(n, 0x3C, np.uint8)
        f = oracle_lib.normalize(oracle_lib.histogram(sym))
        p = oracle_lib.encode_chunk(sym, f)
        assert p.size == 128
        assert np.all(p.view("<u4") == L)


def test_two_symbols_one_bit_each(oracle_lib):
    g = np.random.default_rng(3)
    sym = np.where(g.permutation(65536) < 32768, 0x3C, 0xBC).astype(np.uint8)
    f = oracle_lib.normalize(oracle_lib.histogram(sym))
    assert f[0x3C] == 2048 and f[0xBC] == 2048
    p = oracle_lib.encode_chunk(sym, f)
    W = (p.size - 128) // 2
    # one bit per symbol: 2048 bits per lane, minus what the final state holds
    assert 32 * 127 <= W <= 32 * 128
    assert p.size <= _size_bound(65536, _hq_bits(sym, f))
    out, err = oracle_lib.decode_chunk(p, f, 65536)
    assert err == 0 and np.array_equal(out, sym)


def test_uniform_256_eight_bits_each(oracle_lib):
    g = np.random.default_rng(4)
    sym = g.permutation(np.repeat(np.arange(256, dtype=np.uint8), 256))
    f = oracle_lib.normalize(oracle_lib.histogram(sym))
    assert np.all(f == 16)
    p = oracle_lib.encode_chunk(sym, f)
    W = (p.size - 128) // 2
    assert 32 * 1023 <= W <= 32 * 1024
    assert 65600 <= p.size <= 65664
    out, err = oracle_lib.decode_chunk(p, f, 65536)
    assert err == 0 and np.array_equal(out, sym)


@pytest.mark.parametrize("n", [1, 2, 31, 32, 33, 63, 64, 65, 1000, 65535, 65536])
def test_ragged_lengths(oracle_lib, n):
    g = np.random.default_rng(n)
    sym = (_weights_like(g, n) >> 8).astype(np.uint8)
    f = oracle_lib.normalize(oracle_lib.histogram(sym))
    p = oracle_lib.encode_chunk(sym, f)
    assert p.size % 4 == 0
    states = p[:128].view("<u4")
    if n < 32:
        # lanes that never receive a symbol keep the initial state
        assert np.all(states[n:] == L)
    assert np.all(states >= L)
    assert p.size <= _size_bound(n, _hq_bits(sym, f))
    out, err = oracle_lib.decode_chunk(p, f, n)
    assert err == 0 and np.array_equal(out, sym)


def test_non_palindromic_order(oracle_lib):
    # j mod 251 is not symmetric, so a reversed word or symbol order shows up
    sym = (np.arange(65536) % 251).astype(np.uint8)
    f = oracle_lib.normalize(oracle_lib.histogram(sym))
    p = oracle_lib.encode_chunk(sym, f)
    out, err = oracle_lib.decode_chunk(p, f, 65536)
    assert err == 0 and np.array_equal(out, sym)


def test_every_bf16_pattern_round_trips(oracle_lib):
    v = np.arange(65536, dtype=np.uint16)
    g = np.random.default_rng(11)
    for x in (v, g.permutation(v), np.concatenate([g.permutation(v), v[:12345]])):
        e = oracle_lib.encode(x, "bf16")
        y, err = oracle_lib.decode(e)
        assert err == 0 and np.array_equal(x, y)


def test_seek_is_cumulative_sizes(oracle_lib):
    g = np.random.default_rng(5)
    x = _weights_like(g, 5 * 65536 + 777)
    e = oracle_lib.encode(x, "bf16")
    sizes = []
    for k in range(6):
        sym = (x[65536 * k: 65536 * (k + 1)] >> 8).astype(np.uint8)
        f = oracle_lib.normalize(oracle_lib.histogram(sym))
        assert np.array_equal(f, e.tables[k])
        sizes.append(oracle_lib.encode_chunk(sym, f).size)
    assert np.array_equal(e.seek, np.concatenate([[0], np.cumsum(sizes)]).astype(np.uint64))


def test_entropy_bound_and_excess(oracle_lib):
    """Size within the provable bound of the 12-bit entropy, and in practice
    within 1% of it, on weight-like chunks."""
    g = np.random.default_rng(6)
    for sigma in (0.005, 0.02, 0.05):
        x = _weights_like(g, 65536, sigma)
        sym = (x >> 8).astype(np.uint8)
        f = oracle_lib.normalize(oracle_lib.histogram(sym))
        p = oracle_lib.encode_chunk(sym, f)
        hq = _hq_bits(sym, f)
        assert p.size <= _size_bound(65536, hq)
        assert (p.size - 128) * 8 <= hq * 1.01 + 64


def test_weight_statistics_sanity(oracle_lib):
    """Loose check against the PTWM README's remark that trained weights'
    exponent plane holds ~20 distinct values at ~2.6 bits/byte."""
    from lossless_weight_compression_bf16_amd import synthetic as S
    w = S.workload("bf16-768x2304")
    x = S.tensor_bits(w, 0)
    hi = (x >> 8).astype(np.uint8)
    c = np.bincount(hi, minlength=256)
    p = c[c > 0] / c.sum()
    H = float(-(p * np.log2(p)).sum())
    assert 15 <= (c > 0).sum() <= 40
    assert 2.4 <= H <= 2.9
    e = oracle_lib.encode(x, "bf16")
    total = e.total_bytes
    ratio = total / (2 * x.size)
    assert abs(ratio - (8 + H + 0.079) / 16) < 0.01


def test_corruption_never_crashes(oracle_lib):
    """Flipped bytes, truncation and bad tables give an error or a different
    tensor, never a crash (the decoder bounds every read)."""
    g = np.random.default_rng(9)
    x = _weights_like(g, 3 * 65536 + 100)
    e = oracle_lib.encode(x, "bf16")
    import copy
    detected = 0
    for trial in range(60):
        d = copy.deepcopy(e)
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
        y, err = oracle_lib.decode(d, strict=False)
        if err or not np.array_equal(y, x):
            detected += 1
    assert detected >= 55


# ----------------------------------------------- the state interval [L, 2^32)

@pytest.mark.parametrize("kind", ["weights", "uniform", "rare", "single"])
def test_stored_states_lie_in_the_state_interval(oracle_lib, kind):
    """The encoder keeps every state in [L, 2^32), so the 32 final states it
    stores in front of a chunk are all at least L, whatever the symbols."""
    g = np.random.default_rng(31)
    for n in (1, 33, 4097, 65536):
        if kind == "weights":
            sym = (_weights_like(g, n) >> 8).astype(np.uint8)
        elif kind == "uniform":
            sym = g.integers(0, 256, n).astype(np.uint8)
        elif kind == "rare":  # one frequent symbol, 255 of frequency 1
            sym = np.full(n, 7, np.uint8)
            sym[g.permutation(n)[: min(n, 255)]] = np.arange(min(n, 255)).astype(np.uint8) + 8
        else:
            sym = np.full(n, 200, np.uint8)
        f = oracle_lib.normalize(oracle_lib.histogram(sym))
        st = oracle_lib.encode_chunk(sym, f)[:128].view("<u4")
        assert st.min() >= L, (kind, n)


def test_a_stored_state_below_L_is_rejected(oracle_lib):
    """A chunk whose stored states include one below L is no encoding: the
    decoder reports WCO_EF_BAD_FINAL_STATE, and nothing else, before any
    step; L itself is still accepted (the state of an all-same chunk)."""
    g = np.random.default_rng(32)
    sym = (_weights_like(g, 4096) >> 8).astype(np.uint8)
    f = oracle_lib.normalize(oracle_lib.histogram(sym))
    p = oracle_lib.encode_chunk(sym, f)
    for lane, v in ((0, 0), (5, L - 1), (31, 1)):
        q = p.copy()
        q[4 * lane:4 * lane + 4] = np.frombuffer(np.uint32(v).tobytes(), np.uint8)
        _, err = oracle_lib.decode_chunk(q, f, sym.size)
        assert err == oracle_lib.EF_BAD_FINAL_STATE, (lane, v, err)
    same = np.full(100, 9, np.uint8)
    fs = oracle_lib.normalize(oracle_lib.histogram(same))
    ps = oracle_lib.encode_chunk(same, fs)
    out, err = oracle_lib.decode_chunk(ps, fs, 100)
    assert err == 0 and np.array_equal(out, same)


def _renorm_runs(freq, x, words):
    """Decode steps of one lane from state x, renormalising from `words`;
    returns the per-step renormalisation flags (plain integer arithmetic)."""
    b = np.concatenate([[0], np.cumsum(freq)[:-1]]).astype(np.int64)
    owner = np.repeat(np.arange(256), freq)
    flags = []
    wi = 0
    for _ in range(len(words)):
        slot = x % 4096
        s = owner[slot]
        x = int(freq[s]) * (x >> 12) + slot - int(b[s])
        r = x < L
        if r:
            x = (x << 16) | int(words[wi])
            wi += 1
        flags.append(r)
    return flags


def test_at_most_three_renormalisations_in_a_row():
    """From a state in [L, 2^32) a lane renormalises at most three steps in a
    row (so at most 6 words in 8 steps): the bound the GPU decoder sizes its
    stream ring by.  The adversary below is tight: 255 symbols of frequency
    1, the smallest state L, and words that always land in their slots."""
    freq = np.ones(256, np.int64)
    freq[255] = 4096 - 255
    words = [0] * 64  # slot 0 (symbol 0, frequency 1), smallest high bits
    flags = _renorm_runs(freq, L, words)
    runs, run, best8 = [], 0, 0
    for t, r in enumerate(flags):
        run = run + 1 if r else 0
        runs.append(run)
    for t0 in range(0, len(flags) - 7):
        best8 = max(best8, sum(flags[t0:t0 + 8]))
    assert max(runs) == 3 and best8 == 6
    # random tables, states and words never exceed it
    g = np.random.default_rng(33)
    for trial in range(300):
        k = int(g.integers(1, 257))
        freq = np.zeros(256, np.int64)
        idx = g.choice(256, k, replace=False)
        cut = np.sort(g.choice(np.arange(1, 4096), k - 1, replace=False)) if k > 1 else np.array([], np.int64)
        freq[idx] = np.diff(np.concatenate([[0], cut, [4096]]))
        if trial % 3 == 0:  # many rare symbols
            freq[:] = 1
            freq[int(g.integers(0, 256))] = 4096 - 255
        x = int(g.integers(L, 1 << 32))
        words = g.integers(0, 65536, 96).tolist()
        flags = _renorm_runs(freq, x, words)
        run = 0
        for t, r in enumerate(flags):
            run = run + 1 if r else 0
            assert run <= 3, trial
        for t0 in range(0, len(flags) - 7):
            assert sum(flags[t0:t0 + 8]) <= 6, trial
