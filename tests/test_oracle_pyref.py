"""A second, independent implementation of the chunk coder, written in plain
Python integers one symbol at a time, against the C oracle byte for byte.

The SMEF README's file table and reading order tell of a bug in the order
of its vectorised rANS stream: a coder and a decoder that agree with each
other can still both be wrong about the order.  This module restates the
format's steps (count, normalise to 12 bits, encode 32 interleaved lanes in
reverse, lay out states then words, decode in step and lane order) from
their definition, without looking at how the oracle loops, and requires the
same bytes as the oracle on random tiny inputs of 1 to 5,000 symbols, odd
sizes included, and the oracle's histogram to be numpy's bincount.
"""
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

M = 4096          # 12-bit tables
L = 1 << 16       # state lower bound
LANES = 32


def py_normalize(counts):
    """Largest-remainder rounding to a sum of 4096 that keeps every present
    symbol (count > 0) at frequency >= 1."""
    T = sum(counts)
    f = [0] * 256
    regular = []  # (remainder, symbol) of symbols whose floor is at least 1
    for s, c in enumerate(counts):
        if c == 0:
            continue
        q, r = divmod(c * M, T)
        if q >= 1:
            f[s] = q
            regular.append((r, s))
        else:
            f[s] = 1
    short = M - sum(f)
    if short > 0:
        for _, s in sorted(regular, key=lambda rs: (-rs[0], rs[1]))[:short]:
            f[s] += 1
    while short < 0:
        big = max(range(256), key=lambda s: (f[s], -s))  # largest f, smaller symbol on ties
        f[big] -= 1
        short += 1
    return f


def py_encode(sym, f):
    """States (32 x u32 LE), then the renormalisation words (u16 LE) in the
    order the decoder reads them, then a zero word if their count is odd."""
    start = [0] * 256
    acc = 0
    for s in range(256):
        start[s] = acc
        acc += f[s]
    n = len(sym)
    x = [L] * LANES
    emitted = []  # words in the order the encoder produces them (reverse of reading)
    for j in range(n - 1, -1, -1):  # the last symbol first: step descending, lane descending
        lane = j % LANES
        s = sym[j]
        if x[lane] >= f[s] << 20:
            emitted.append(x[lane] & 0xFFFF)
            x[lane] >>= 16
        x[lane] = (x[lane] // f[s]) * M + x[lane] % f[s] + start[s]
    words = emitted[::-1]
    if len(words) % 2:
        words.append(0)
    return struct.pack(f"<{LANES}I", *x) + struct.pack(f"<{len(words)}H", *words)


def py_decode(payload, f, n):
    """Symbols, or None when the stream is not one the encoder can produce."""
    if sum(f) != M or len(payload) < 128 or len(payload) % 4:
        return None
    owner = []
    start = [0] * 256
    acc = 0
    for s in range(256):
        start[s] = acc
        owner += [s] * f[s]
        acc += f[s]
    x = list(struct.unpack_from(f"<{LANES}I", payload, 0))
    if any(v < L for v in x):  # the stored final states lie in [L, 2^32)
        return None
    pos = 128
    out = []
    for j in range(n):  # step ascending, lane ascending
        lane = j % LANES
        slot = x[lane] % M
        s = owner[slot]
        out.append(s)
        x[lane] = f[s] * (x[lane] // M) + slot - start[s]
        if x[lane] < L:
            if pos + 2 > len(payload):
                return None
            x[lane] = (x[lane] << 16) | struct.unpack_from("<H", payload, pos)[0]
            pos += 2
    left = len(payload) - pos
    if any(v != L for v in x) or left not in (0, 2):
        return None
    if left == 2 and payload[pos:] != b"\0\0":
        return None
    return out


def _symbols(g, kind, n):
    if kind == "weights":  # the coded byte of N(0, 0.02) weights rounded to BF16
        v = (g.standard_normal(n) * 0.02).astype(np.float32).view(np.uint32)
        return ((v + 0x7FFF + ((v >> 16) & 1)) >> 24).astype(np.uint8)
    if kind == "uniform":
        return g.integers(0, 256, n).astype(np.uint8)
    if kind == "few":
        return g.choice(np.array([3, 200, 201, 77], np.uint8), n, p=[0.7, 0.2, 0.09, 0.01])
    if kind == "one":
        return np.full(n, int(g.integers(0, 256)), np.uint8)
    if kind == "rare":  # many symbols seen once or twice: the table's excess case
        base = np.full(n, 128, np.uint8)
        k = min(n, 240)
        base[g.choice(n, k, replace=False)] = g.choice(np.arange(256, dtype=np.uint8), k)
        return base
    raise ValueError(kind)


KINDS = ["weights", "uniform", "few", "one", "rare"]


def _cases():
    g = np.random.default_rng(2024)
    out = []
    for i in range(60):
        n = int(g.integers(1, 5001))
        if i % 3 == 0:
            n |= 1  # odd sizes
        out.append((KINDS[i % len(KINDS)], n, 1000 + i))
    return out + [("weights", 1, 7), ("uniform", 31, 8), ("few", 33, 9), ("weights", 64, 10)]


@pytest.mark.parametrize("kind,n,seed", _cases())
def test_same_bytes_as_the_oracle(oracle_lib, kind, n, seed):
    g = np.random.default_rng(seed)
    sym = _symbols(g, kind, n)
    counts = [int(c) for c in np.bincount(sym, minlength=256)]
    f_py = py_normalize(counts)
    f_or = oracle_lib.normalize(oracle_lib.histogram(sym))
    assert f_py == [int(v) for v in f_or]
    p_py = py_encode([int(s) for s in sym], f_py)
    p_or = oracle_lib.encode_chunk(sym, f_or).tobytes()
    assert p_py == p_or
    # each side decodes the other's bytes
    assert py_decode(p_or, f_py, n) == [int(s) for s in sym]
    d, err = oracle_lib.decode_chunk(np.frombuffer(p_py, np.uint8), f_or, n)
    assert err == 0 and np.array_equal(d, sym)


def test_non_palindromic_sequence(oracle_lib):
    """s_j = j mod 251: reversing steps, lanes or words changes the bytes."""
    sym = (np.arange(4099) % 251).astype(np.uint8)
    f = py_normalize([int(c) for c in np.bincount(sym, minlength=256)])
    p = py_encode([int(s) for s in sym], f)
    assert p == oracle_lib.encode_chunk(sym, np.array(f, np.uint16)).tobytes()
    assert py_decode(p, f, sym.size) == [int(s) for s in sym]


def test_normalisation_of_large_histograms(oracle_lib):
    """Chunk-sized totals with a shortfall, an excess (many forced symbols)
    and ties in the remainders."""
    g = np.random.default_rng(77)
    for trial in range(200):
        T = int(g.integers(1, 65537))
        k = int(g.integers(1, 257))
        support = g.choice(256, k, replace=False)
        if trial % 2:  # one dominant symbol and many seen once: sum of floors exceeds 4096
            c = np.zeros(256, np.int64)
            c[support] = 1
            c[support[0]] += max(T - k, 0)
        else:
            c = np.bincount(g.choice(support, T), minlength=256)
        counts = [int(v) for v in c]
        assert py_normalize(counts) == [int(v) for v in oracle_lib.normalize(np.array(counts, np.uint32))]


def test_histogram_is_bincount(oracle_lib):
    g = np.random.default_rng(5)
    for n in (1, 2, 255, 256, 4097, 65535, 65536):
        for sym in (g.integers(0, 256, n).astype(np.uint8), np.full(n, 255, np.uint8),
                    _symbols(g, "weights", n)):
            assert np.array_equal(oracle_lib.histogram(sym), np.bincount(sym, minlength=256))


HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_decoder_under_address_and_ub_sanitizers(tmp_path):
    """The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
    (host code only) decodes thousands of corrupted streams -- flipped bits,
    truncations, inflated table entries, moved seek entries, BF16 and FP32
    -- and every one ends in an error or a different tensor, with no
    out-of-bounds access and no undefined arithmetic."""
    exe = tmp_path / "oracle_fuzz"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-pthread", "-I", os.path.join(ROOT, "oracle"),
           os.path.join(HERE, "oracle_fuzz.c"), os.path.join(ROOT, "oracle", "wc_oracle.c"), "-o", str(exe)]
    b = subprocess.run(cmd, capture_output=True, text=True)
    if b.returncode != 0 and "asan" in (b.stderr + b.stdout).lower():
        pytest.skip("this gcc has no sanitizer runtime")
    assert b.returncode == 0, b.stderr
    # a library preloaded into every process may precede the ASan runtime;
    # ASan is told not to insist on coming first
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe), "2100"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
    detected, trials = (int(v) for v in r.stdout.split()[-2:])
    assert trials == 2100 and detected >= 0.9 * trials
