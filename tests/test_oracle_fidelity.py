"""Pins of the oracle's mask-fidelity diagnostic: the true block mass of dense
attention and the recall of a mask against the top-mass blocks (review record of
arXiv 2507.13546, the referee's per-block fidelity test)."""

import itertools

import numpy as np
import torch

import oracle


def _qk(seed, BH, S, D, spread=1.0):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((BH, S, D)) * spread).astype(np.float32)
    k = (rng.standard_normal((BH, S, D)) * spread).astype(np.float32)
    return q, k


def test_rows_are_distributions():
    q, k = _qk(0, 2, 512, 16, 1.5)
    m = oracle.block_mass(q, k, 64)
    assert m.shape == (2, 8, 8)
    np.testing.assert_allclose(m.sum(axis=-1), 1.0, atol=1e-12)
    assert (m >= 0).all()


def test_n1_is_the_token_softmax():
    q, k = _qk(1, 1, 48, 8, 1.2)
    m = oracle.block_mass(q, k, 1)
    qt, kt = torch.from_numpy(q).double(), torch.from_numpy(k).double()
    p = torch.softmax(qt @ kt.transpose(1, 2) / np.sqrt(8), dim=-1).numpy()
    np.testing.assert_allclose(m, p, rtol=1e-12, atol=1e-15)


def test_equals_attention_output_on_block_indicator_values():
    # With V = one-hot of each key's block, dense attention's output for token s is
    # the vector of its block masses; M averages it over the block's queries. The
    # attention oracle is pinned separately (SDPA, finite differences).
    BH, S, D, N = 2, 384, 8, 64
    n = S // N
    q, k = _qk(2, BH, S, D, 2.0)
    v = np.zeros((BH, S, D), dtype=np.float32)
    for u in range(S):
        v[:, u, u // N] = 1.0
    o, _ = oracle.attn_fwd(q, k, v, np.ones((BH, n, n), dtype=np.uint8), N)
    want = o[:, :, :n].reshape(BH, n, N, n).mean(axis=2)
    np.testing.assert_allclose(oracle.block_mass(q, k, N), want, rtol=1e-10, atol=1e-13)


def test_invariances():
    q, k = _qk(3, 1, 256, 8, 1.5)
    m = oracle.block_mass(q, k, 64)
    # a common shift of every key adds a per-row constant to the logits
    shift = np.random.default_rng(4).standard_normal(8).astype(np.float32)
    np.testing.assert_allclose(oracle.block_mass(q, k + shift, 64), m, rtol=1e-5, atol=1e-9)
    # shuffling tokens inside key blocks changes nothing; permuting key blocks permutes columns
    perm_in = np.concatenate([64 * b + np.random.default_rng(b).permutation(64) for b in range(4)])
    np.testing.assert_allclose(oracle.block_mass(q, k[:, perm_in], 64), m, rtol=1e-12, atol=1e-15)
    bp = np.array([2, 0, 3, 1])
    perm_blk = np.concatenate([np.arange(64 * b, 64 * b + 64) for b in bp])
    np.testing.assert_allclose(oracle.block_mass(q, k[:, perm_blk], 64), m[:, :, bp], rtol=1e-12,
                               atol=1e-15)
    # identical keys: uniform attention, every block holds 1/n
    kk = np.repeat(k[:, :1], 256, axis=1)
    np.testing.assert_allclose(oracle.block_mass(q, kk, 64), 0.25, atol=1e-12)


def test_block_subset_matches_full():
    q, k = _qk(5, 2, 320, 8)
    full = oracle.block_mass(q, k, 64)
    sub = oracle.block_mass(q, k, 64, blocks=[1, 7, 9])
    for b in (1, 7, 9):
        np.testing.assert_array_equal(sub[b // 5, b % 5], full[b // 5, b % 5])
    assert np.isnan(sub[0, 0]).all()


def test_recall_keep_all_and_brute_force_best():
    rng = np.random.default_rng(6)
    n = 7
    raw = rng.random((3, n, n)) ** 3
    mass = raw / raw.sum(axis=-1, keepdims=True)
    mask = (rng.random((3, n, n)) < 0.4).astype(np.uint8)
    mask[..., 0] = 1
    rec, best = oracle.mask_recall(mass, mask)
    for b in range(3):
        for i in range(n):
            c = int(mask[b, i].sum())
            brute = max(sum(mass[b, i, list(s)]) for s in itertools.combinations(range(n), c))
            assert abs(best[b, i] - brute) < 1e-12
            assert abs(rec[b, i] - mass[b, i][mask[b, i] == 1].sum()) < 1e-12
            assert rec[b, i] <= best[b, i] + 1e-15
    r1, b1 = oracle.mask_recall(mass, np.ones_like(mask))
    np.testing.assert_allclose(r1, 1.0, atol=1e-12)
    np.testing.assert_allclose(b1, 1.0, atol=1e-12)
    # the top-mass mask reaches its own bound
    c = mask.sum(axis=-1)
    top = np.zeros_like(mask)
    order = np.argsort(-mass, axis=-1, kind="stable")
    for b in range(3):
        for i in range(n):
            top[b, i, order[b, i, :c[b, i]]] = 1
    rt, bt = oracle.mask_recall(mass, top)
    np.testing.assert_allclose(rt, bt, atol=1e-12)
