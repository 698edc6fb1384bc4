"""Pins of the oracle's 12-bit table normalisation.

The pages name rANS but give no table construction; the construction used
(largest-remainder rounding with a zero guard and a largest-first fix-up) is
pinned here by hand-derived cases (tests/golden/normalize_cases.json), by an
independent closed form of the fix-up loop, and by brute force over tiny
alphabets.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "normalize_cases.json")


def _expand(case):
    counts = np.zeros(256, np.uint32)
    expect = np.zeros(256, np.int64)
    for k, v in case["counts"].items():
        if k == "all":
            counts[:] = v
        else:
            counts[int(k)] = v
    for k, v in case["expect"].items():
        if k == "all":
            expect[:] = v
        else:
            expect[int(k)] = v
    rare = case.get("rare")
    if rare == "every symbol except 60":
        idx = [s for s in range(256) if s != 60]
    elif rare == "symbols 0..99 except 60":
        idx = [s for s in range(100) if s != 60]
    else:
        idx = []
    for s in idx:
        counts[s] = 1
        expect[s] = case["expect_rare"]
    return counts, expect


def _cases():
    with open(GOLDEN) as fh:
        return json.load(fh)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_golden_tables(oracle_lib, case):
    counts, expect = _expand(case)
    assert counts.sum() <= 65536
    f = oracle_lib.normalize(counts)
    assert np.array_equal(f.astype(np.int64), expect), case["derivation"]


def _fixup_closed_form(f0, excess):
    """Result of 'excess' times 'decrement the largest f, smallest symbol on
    ties', written as a water level: every f is cut to v+1, where v is the
    largest level whose cut costs at least 'excess', and the remaining
    decrements take the smallest symbols sitting at v+1 down to v."""
    f0 = np.asarray(f0, np.int64)

    def cost(v):
        return int(np.maximum(f0 - v, 0).sum())

    v = int(f0.max())
    while cost(v) < excess:
        v -= 1
    f = np.minimum(f0, v + 1)
    left = excess - cost(v + 1)
    for s in np.nonzero(f0 >= v + 1)[0][:left]:
        f[s] = v
    return f


def _raw_stage(counts):
    T = int(counts.sum())
    c = counts.astype(np.int64)
    q = c * 4096 // T
    f = np.where(c > 0, np.maximum(q, 1), 0)
    return T, c, q, f


def test_properties_random(oracle_lib):
    """Sum, support, rounding distance, remainder order, and the fix-up's
    closed form, on many random histograms (normal-like and heavy-tailed)."""
    g = np.random.default_rng(7)
    for trial in range(400):
        T = int(g.integers(1, 65537))
        k = int(g.integers(1, 257))
        if trial % 3 == 0:
            p = g.dirichlet(np.full(k, 0.05))        # very skewed: many forced symbols
        elif trial % 3 == 1:
            p = g.dirichlet(np.ones(k))
        else:
            p = np.full(k, 1.0 / k)
        sym = g.choice(256, k, replace=False)
        counts = np.zeros(256, np.uint32)
        np.add.at(counts, sym[g.choice(k, T, p=p)], 1)
        f = oracle_lib.normalize(counts).astype(np.int64)
        T, c, q, fr = _raw_stage(counts)
        assert f.sum() == 4096
        assert np.array_equal(f > 0, c > 0)
        D = 4096 - int(fr.sum())
        if D >= 0:
            regular = q >= 1
            # each regular f is q or q+1; forced ones stay 1
            assert np.all((f[regular] == q[regular]) | (f[regular] == q[regular] + 1))
            assert np.all(f[(c > 0) & ~regular] == 1)
            assert np.all(np.abs(f[regular] - c[regular] * 4096 / T) < 1)
            up = regular & (f == q + 1)
            down = regular & (f == q)
            if up.any() and down.any():
                r = c * 4096 % T
                # nothing left behind ranks before anything that got +1
                worst_up = min(zip(-r[up], np.nonzero(up)[0]), key=lambda t: (-t[0], -t[1]))
                best_down = min(zip(-r[down], np.nonzero(down)[0]))
                assert worst_up < best_down
        else:
            assert np.array_equal(f, _fixup_closed_form(fr, -D))


def _hq(c, f):
    return sum(ci * math.log2(4096 / fi) for ci, fi in zip(c, f) if ci)


def test_brute_force_three_symbols(oracle_lib):
    """Every count vector with T <= 8 over three symbols: the table is
    valid, and its cost H_q is within 0.01 bit/symbol of the best split of
    4096.  The best split is found by exhaustive search over a window of
    +-96 around the ideal c*4096/T; H_q is separable and convex in f, so the
    integer optimum lies within one step of the real one, well inside the
    window."""
    worst_gap = 0.0
    for T in range(1, 9):
        for c1 in range(T + 1):
            for c2 in range(T + 1 - c1):
                c3 = T - c1 - c2
                counts = np.zeros(256, np.uint32)
                counts[[3, 100, 250]] = [c1, c2, c3]
                f = oracle_lib.normalize(counts).astype(np.int64)
                assert f.sum() == 4096
                assert np.array_equal(f > 0, counts > 0)
                cs = np.array([c1, c2, c3], np.float64)
                got = _hq(cs, f[[3, 100, 250]])
                present = np.nonzero(cs)[0]
                if present.size == 1:
                    best = 0.0
                else:
                    ideal = cs[present] * 4096 / T
                    axes = [np.arange(max(1, int(v) - 96), min(4095, int(v) + 97))
                            for v in ideal[:-1]]
                    grid = np.stack(np.meshgrid(*axes, indexing="ij"), -1).reshape(-1, len(axes))
                    last = 4096 - grid.sum(1)
                    ok = last >= 1
                    full = np.concatenate([grid[ok], last[ok, None]], 1).astype(np.float64)
                    best = float((cs[present] * np.log2(4096 / full)).sum(1).min())
                gap = (got - best) / T
                worst_gap = max(worst_gap, gap)
                assert gap < 0.01, (cs, f[[3, 100, 250]], got, best)
    assert worst_gap >= 0.0
