"""Pins of the oracle's tile order and BF16 GEMM (row f3: decode fused with
its consumer).

The tile order is this library's own permutation (not the pages'); what it
must achieve is fixed by the matrix instruction it feeds: with AMD's
documented operand layout of v_mfma_f32_16x16x16_bf16 (wave lane L = 16 j +
i: A[i][4j..4j+3], B[4j..4j+3][i], D[4j..4j+3][i]), the values a decoder half
holds at the end of a group, exchanged between halves as the kernel does,
must make the instruction compute X W^T for the tile.  A numpy model of the
instruction checks that here, so a wrong index in the order fails.  The GEMM
reference is pinned to exact rational arithmetic and closed forms.
"""
from fractions import Fraction

import numpy as np
import pytest


def _bf16(x):
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)  # round to nearest even


def _val(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32).astype(np.float64)


def test_tile_order_is_a_permutation_and_inverts(oracle_lib):
    for rows, cols in [(16, 16), (32, 48), (48, 2048 + 16), (16 * 5, 16 * 7)]:
        idx = np.arange(rows * cols, dtype=np.uint32)
        # values = index modulo 2^16 plus a second pass on the high part keeps it a bijection check
        lo = (idx & 0xFFFF).astype(np.uint16).reshape(rows, cols)
        hi = (idx >> 16).astype(np.uint16).reshape(rows, cols)
        tl, th = oracle_lib.tile_order(lo), oracle_lib.tile_order(hi)
        back = (th.astype(np.uint32) << 16) | tl
        assert np.array_equal(np.sort(back), idx)
        assert np.array_equal(oracle_lib.tile_order(tl, True, (rows, cols)), lo)


def test_tile_order_rejects_ragged_shapes(oracle_lib):
    with pytest.raises(ValueError):
        oracle_lib.tile_order(np.zeros((16, 24), np.uint16))
    with pytest.raises(ValueError):
        oracle_lib.tile_order(np.zeros((8, 16), np.uint16))


def test_tiles_run_panel_by_panel(oracle_lib):
    # tile t of a rows x cols matrix holds rows 16 (t div cols/16) .. +15 and
    # columns 16 (t mod cols/16) .. +15, whatever the order inside the tile
    rows, cols = 48, 80
    r, c = np.meshgrid(np.arange(rows), np.arange(cols), indexing="ij")
    tr = oracle_lib.tile_order(r.astype(np.uint16)).reshape(-1, 256)
    tc = oracle_lib.tile_order(c.astype(np.uint16)).reshape(-1, 256)
    for t in range(tr.shape[0]):
        p, b = divmod(t, cols // 16)
        assert sorted(set(tr[t])) == list(range(16 * p, 16 * p + 16))
        assert sorted(set(tc[t])) == list(range(16 * b, 16 * b + 16))


def _mfma_16x16x16(a_lanes, b_lanes):
    """The instruction by its documented operand layout: a_lanes, b_lanes
    (64 x 4) -> D lanes (64 x 4) with D = A B."""
    A = np.zeros((16, 16))
    Bm = np.zeros((16, 16))
    for L in range(64):
        i, j = L % 16, L // 16
        A[i, 4 * j:4 * j + 4] = a_lanes[L]
        Bm[4 * j:4 * j + 4, i] = b_lanes[L]
    D = A @ Bm
    return np.array([D[4 * (L // 16):4 * (L // 16) + 4, L % 16] for L in range(64)])


def _b_lanes_of_half(v, half):
    """B operand lanes for the tile that decoder half `half` holds (v: its 256
    tile-ordered values; lane l of the half holds v[8l .. 8l+7]): the half
    keeps 4 values per lane and sends the other 4 to the other half."""
    b = np.zeros((64, 4))
    for L in range(64):
        l = L % 32
        first = (L < 32)  # wave lanes 0-31 take elements 0-3 of lane l, 32-63 elements 4-7
        b[L] = v[8 * l:8 * l + 4] if first else v[8 * l + 4:8 * l + 8]
    return b


@pytest.mark.parametrize("half", [0, 1])
def test_tile_order_feeds_the_matrix_instruction(oracle_lib, half):
    g = np.random.default_rng(7 + half)
    rows, cols = 32, 64
    w = g.integers(-8, 8, (rows, cols)).astype(np.float64)
    x = g.integers(-8, 8, (16, cols)).astype(np.float64)
    wb = _bf16(w.astype(np.float32))
    t = _val(oracle_lib.tile_order(wb)).reshape(-1, 256)
    for ti in range(t.shape[0]):
        p, kb = divmod(ti, cols // 16)
        a = np.array([x[L % 16, 16 * kb + 4 * (L // 16):16 * kb + 4 * (L // 16) + 4] for L in range(64)])
        d = _mfma_16x16x16(a, _b_lanes_of_half(t[ti], half))
        want = x[:, 16 * kb:16 * kb + 16] @ w[16 * p:16 * p + 16, 16 * kb:16 * kb + 16].T
        got = np.zeros((16, 16))
        for L in range(64):
            got[4 * (L // 16):4 * (L // 16) + 4, L % 16] = d[L]
        assert np.array_equal(got, want), ti


def test_gemm_exact_on_small_integers_and_fractions(oracle_lib):
    g = np.random.default_rng(3)
    m, n, k = 3, 5, 7
    # values in [0.5, 4): every product and partial sum is exact in double
    x = _bf16((g.random((m, k)) * 3.5 + 0.5).astype(np.float32) * np.where(g.random((m, k)) < 0.5, -1, 1))
    w = _bf16((g.random((n, k)) * 3.5 + 0.5).astype(np.float32) * np.where(g.random((n, k)) < 0.5, -1, 1))
    y, mag = oracle_lib.gemm_bf16(x, w, magnitude=True)
    xv, wv = _val(x), _val(w)
    for i in range(m):
        for j in range(n):
            exact = sum(Fraction(float(xv[i, t])) * Fraction(float(wv[j, t])) for t in range(k))
            assert Fraction(float(y[i, j])) == exact
            assert Fraction(float(mag[i, j])) == sum(abs(Fraction(float(xv[i, t])) * Fraction(float(wv[j, t])))
                                                     for t in range(k))


def test_gemm_closed_forms(oracle_lib):
    k = 2048
    one = np.full((4, k), 0x3F80, np.uint16)  # BF16 1.0
    y = oracle_lib.gemm_bf16(one, np.full((6, k), 0x3F80, np.uint16))
    assert np.all(y == k)
    # a one-hot row of X picks one column of W (W not transposed: y[0][j] = w[j][5])
    g = np.random.default_rng(1)
    w = _bf16(g.standard_normal((8, 32)).astype(np.float32))
    x = np.zeros((1, 32), np.uint16)
    x[0, 5] = 0x3F80
    assert np.array_equal(oracle_lib.gemm_bf16(x, w)[0], _val(w[:, 5]))
    # -2.0 (0xC000) times 0.5 (0x3F00) is -1 per term
    assert np.all(oracle_lib.gemm_bf16(np.full((1, 3), 0xC000, np.uint16), np.full((2, 3), 0x3F00, np.uint16)) == -3)


def test_gemm_rejects_mismatched_inner_dimension(oracle_lib):
    with pytest.raises(ValueError):
        oracle_lib.gemm_bf16(np.zeros((2, 3), np.uint16), np.zeros((2, 4), np.uint16))
