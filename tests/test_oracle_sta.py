"""Pins of the oracle's STA block map (section 2.2 eq. (4)-(5), section 3.1.3)."""

import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dim_count(L, w):
    """Number of (query, key) coordinate pairs on one axis for a clipped centred window."""
    lo, hi = (w - 1) // 2, w // 2
    return sum(min(L - 1, c + hi) - max(0, c - lo) + 1 for c in range(L))


def test_sta_count_is_product_of_axis_counts():
    for (T, Hs, Ws, wt, wh, ww) in [(4, 16, 16, 3, 8, 8), (11, 32, 32, 11, 24, 24),
                                    (5, 24, 40, 2, 16, 24), (3, 8, 8, 1, 8, 8)]:
        P = 8
        m = oracle.sta_mask(T, Hs, Ws, P, wt, wh, ww)
        exp = _dim_count(T, wt) * _dim_count(Hs // P, wh // P) * _dim_count(Ws // P, ww // P)
        assert int(m.sum()) == exp


def test_sta_interior_rows_follow_eq5():
    # Eq. (5): a query tile whose window fits the grid keeps
    # (W_T/B_T)(W_H/B_H)(W_W/B_W) key tiles.
    T, Hs, Ws, P = 21, 48, 80, 8
    for (wt, wh, ww) in [(18, 40, 40), (11, 24, 24), (11, 40, 40), (4, 16, 16)]:
        m = oracle.sta_mask(T, Hs, Ws, P, wt, wh, ww)
        tH, tW = Hs // P, Ws // P
        lo = lambda w: (w - 1) // 2
        hi = lambda w: w // 2
        interior = 0
        for i in range(m.shape[0]):
            t, y, x = i // (tH * tW), (i // tW) % tH, i % tW
            if (t - lo(wt) >= 0 and t + hi(wt) < T and y - lo(wh // P) >= 0 and y + hi(wh // P) < tH
                    and x - lo(ww // P) >= 0 and x + hi(ww // P) < tW):
                interior += 1
                assert m[i].sum() == wt * (wh // P) * (ww // P)
        assert interior > 0


def test_sta_reproduces_table1_sparsities():
    with open(os.path.join(GOLDEN, "table1_sta.json")) as f:
        g = json.load(f)
    grid = g["grid"]
    for row in g["rows"]:
        m = oracle.sta_mask(grid["T"], grid["Hs"], grid["Ws"], grid["P"], *row["window"])
        sparsity = 100.0 * (1.0 - m.mean())
        assert abs(sparsity - row["paper_sparsity_pct"]) <= g["tolerance_pct_points"], row


def test_sta_exact_values_on_720p_grid():
    # The clipped reading gives exactly these on the 21 x 48 x 80 grid.
    m1 = oracle.sta_mask(21, 48, 80, 8, 18, 40, 40)
    m2 = oracle.sta_mask(21, 48, 80, 8, 18, 24, 24)
    assert int(m1.sum()) == 313632 and int(m2.sum()) == 133056
    assert m1.shape == (1260, 1260)


def test_sta_union_workload_counts():
    # 11 frames x 3x3 tiles on the 11 x 32 x 32 grid: 91 x 10 x 10 kept pairs,
    # 24 to 99 key blocks per query block.
    m = oracle.sta_mask(11, 32, 32, 8, 11, 24, 24)
    assert int(m.sum()) == 9100
    rows = m.sum(1)
    assert rows.min() == 24 and rows.max() == 99


def test_sta_symmetric_for_odd_windows_and_full_for_huge_windows():
    m = oracle.sta_mask(7, 40, 40, 8, 5, 24, 40)
    np.testing.assert_array_equal(m, m.T)
    full = oracle.sta_mask(4, 16, 24, 8, 8, 32, 48)
    assert full.all()
    diag = oracle.sta_mask(4, 16, 24, 8, 1, 8, 8)
    np.testing.assert_array_equal(diag, np.eye(diag.shape[0], dtype=np.uint8))


def test_union_contains_both_operands():
    rng = np.random.default_rng(3)
    n = 4 * 2 * 2
    nab = (rng.random((2, n, n)) < 0.2).astype(np.uint8)
    sta = oracle.sta_mask(4, 16, 16, 8, 3, 8, 8)
    u = oracle.union(nab, sta)
    assert np.all(u >= nab) and np.all(u >= sta[None])
    np.testing.assert_array_equal(u, np.maximum(nab, sta[None]))
