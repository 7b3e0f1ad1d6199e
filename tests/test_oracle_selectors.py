"""Pins of the oracle's variant selectors: Top-k blocks and the STA-only static mask.

Top-k is the fixed-budget selector the CDF rule is compared with (review record of
arXiv 2507.13546, referee comment on Appendix C); STA-only is Table 1's static
baseline (section 2.2, eq. (4)-(5)).
"""

import json
import os

import numpy as np
import pytest
from scipy.stats import rankdata

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "topk_rows.json")


def _softmax_rows(rng, BH, n, spread=3.0):
    x = rng.standard_normal((BH, n, n)) * spread
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def test_count_above_matches_library_ranks():
    rng = np.random.default_rng(0)
    a = _softmax_rows(rng, 3, 17)
    # ties: quantise one head's rows to a few levels
    a[1] = np.round(a[1] * 8) / 8
    c = oracle.count_above(a)
    for bh in range(3):
        for i in range(17):
            want = rankdata(-a[bh, i], method="min") - 1   # entries strictly larger
            np.testing.assert_array_equal(c[bh, i], want)


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: f"k{c['k']}_{c['p']}")
def test_topk_golden_rows(case):
    a = np.asarray(case["p"], dtype=np.float64)[None, None, :].repeat(4, axis=1)
    m = oracle.topk_mask(a, case["k"])
    np.testing.assert_array_equal(m[0, 0], case["expected"])


def test_topk_distinct_rows_keep_exactly_the_k_largest():
    rng = np.random.default_rng(1)
    a = _softmax_rows(rng, 2, 23)
    for k in (1, 2, 5, 22, 23, 40):
        m = oracle.topk_mask(a, k)
        assert np.all(m.sum(axis=-1) == min(k, 23))
        for bh in range(2):
            for i in range(23):
                top = np.argsort(-a[bh, i], kind="stable")[: min(k, 23)]
                assert set(np.nonzero(m[bh, i])[0]) == set(top)


def test_topk_invariants():
    rng = np.random.default_rng(2)
    a = _softmax_rows(rng, 2, 19)
    a[0, :5] = np.round(a[0, :5] * 4) / 4                    # rows with ties
    prev = np.zeros_like(a, dtype=np.uint8)
    for k in range(1, 21):
        m = oracle.topk_mask(a, k)
        assert np.all(m >= prev)                              # nested in k
        assert np.all(m.sum(axis=-1) >= min(k, 19))           # at least k (ties add)
        prev = m
    m1 = oracle.topk_mask(a, 1)
    assert np.all(m1[np.arange(2)[:, None], np.arange(19)[None, :], a.argmax(-1)] == 1)
    perm = rng.permutation(19)                                # equivariance
    np.testing.assert_array_equal(oracle.topk_mask(a[:, :, perm], 4), oracle.topk_mask(a, 4)[:, :, perm])
    with pytest.raises(ValueError):
        oracle.topk_mask(a, 0)


def test_topk_with_the_cdf_count_is_the_cdf_mask():
    # On rows without ties the CDF rule keeps a prefix of the descending order, so
    # it equals Top-k with k = the number of blocks it keeps in that row.
    rng = np.random.default_rng(3)
    a = _softmax_rows(rng, 2, 31)
    for thr in (0.1, 0.5, 0.8, 0.95):
        cdf = oracle.cdf_mask(oracle.mass_above(a), thr)
        counts = cdf.sum(axis=-1)
        for bh in range(2):
            for i in range(31):
                row = oracle.topk_mask(a[bh:bh + 1, :, :], int(counts[bh, i]))[0, i]
                np.testing.assert_array_equal(row, cdf[bh, i])


def test_build_topk_mask_chain_and_union():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 2, 4 * 16 * 16, 8)).astype(np.float32)
    k = rng.standard_normal((1, 2, 4 * 16 * 16, 8)).astype(np.float32)
    sta = dict(T=4, Hs=16, Ws=16, P=8, win_t=1, win_h=8, win_w=8)
    res = oracle.build_topk_mask(q, k, 64, 3, sta=sta)
    assert np.all(res["mask_topk"].sum(axis=-1) >= 3)
    s = oracle.sta_mask(**sta)
    assert np.all(res["mask"] >= res["mask_topk"]) and np.all(res["mask"] >= s[None])
    np.testing.assert_array_equal(res["mask"], np.maximum(res["mask_topk"], s[None]))
    # the same chain through the CDF path's pieces
    a = oracle.reduced_map(oracle.pool(q, 64), oracle.pool(k, 64), 1 / np.sqrt(8))
    np.testing.assert_array_equal(res["mask_topk"], oracle.topk_mask(a, 3))


def test_sta_only_mask_is_the_window_for_every_head():
    m = oracle.sta_only_mask(3, 4, 16, 24, 8, 3, 8, 16)
    s = oracle.sta_mask(4, 16, 24, 8, 3, 8, 16)
    assert m.shape == (3,) + s.shape
    for h in range(3):
        np.testing.assert_array_equal(m[h], s)
