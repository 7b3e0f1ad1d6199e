"""Pins of the oracle's mask stage (pooling, reduced softmax, CDF selection).

Each test checks the oracle against something fixed independently of its code:
a library routine, the paper's Algorithm 1 executed literally with numpy's sort
and cumulative sum, an exhaustive subset search, hand-worked rows, or an
invariant the mathematics forces.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


# ---------------------------------------------------------------- pooling
def test_pool_equals_library_average_pool():
    x = _rand((3, 256, 24), 1)
    got = oracle.pool(x, 16)
    ref = torch.nn.functional.avg_pool1d(
        torch.from_numpy(x).double().transpose(1, 2), kernel_size=16).transpose(1, 2).numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def test_pool_block_size_one_is_identity_and_constant_blocks():
    x = _rand((2, 64, 8), 2)
    np.testing.assert_array_equal(oracle.pool(x, 1), x.astype(np.float64))
    c = np.repeat(_rand((2, 4, 8), 3), 16, axis=1)  # every block constant
    np.testing.assert_allclose(oracle.pool(c, 16), c[:, ::16].astype(np.float64), atol=1e-14)


# ---------------------------------------------------------------- reduced map
def test_reduced_map_with_unit_blocks_is_token_softmax():
    # N = 1: the reduced map is the full token attention matrix of eq. (2).
    q, k = _rand((2, 48, 16), 4), _rand((2, 48, 16), 5)
    a = oracle.reduced_map(oracle.pool(q, 1), oracle.pool(k, 1), 1.0 / math.sqrt(16))
    ref = torch.softmax(torch.from_numpy(q).double() @ torch.from_numpy(k).double().transpose(1, 2)
                        / math.sqrt(16), dim=-1).numpy()
    np.testing.assert_allclose(a, ref, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(a.sum(-1), 1.0, atol=1e-12)


def test_reduced_map_of_pooled_blocks_matches_library_chain():
    q, k = _rand((2, 512, 32), 6), _rand((2, 512, 32), 7)
    qa = torch.nn.functional.avg_pool1d(torch.from_numpy(q).double().transpose(1, 2), 64).transpose(1, 2)
    ka = torch.nn.functional.avg_pool1d(torch.from_numpy(k).double().transpose(1, 2), 64).transpose(1, 2)
    ref = torch.softmax(qa @ ka.transpose(1, 2) / math.sqrt(32), dim=-1).numpy()
    a = oracle.build_mask(q, k, 64, 1.0)["a"]
    np.testing.assert_allclose(a, ref, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- selection
def _alg1_literal(p, thr):
    """Algorithm 1 steps 8-11 with numpy: ascending stable sort, cumsum, >=, scatter back."""
    order = np.argsort(p, axis=-1, kind="stable")
    vals = np.take_along_axis(p, order, axis=-1)
    cvals = np.cumsum(vals, axis=-1)
    m_sorted = cvals >= 1.0 - thr
    out = np.zeros_like(m_sorted)
    np.put_along_axis(out, order, m_sorted, axis=-1)
    return out, order, cvals


def _random_probs(BH, n, seed, temp=3.0):
    logits = np.random.default_rng(seed).standard_normal((BH, n, n)) * temp
    e = np.exp(logits - logits.max(-1, keepdims=True))
    return e / e.sum(-1, keepdims=True)


@pytest.mark.parametrize("thr", [0.05, 0.2, 0.5, 0.7, 0.9, 0.99])
def test_selection_matches_literal_algorithm1(thr):
    p = _random_probs(3, 40, 11)
    got = oracle.cdf_mask(oracle.mass_above(p), thr).astype(bool)
    ref, order, cvals = _alg1_literal(p, thr)
    # Entries whose cumulative sum sits within rounding of 1 - thr are excused.
    near = np.zeros_like(ref)
    np.put_along_axis(near, order, np.abs(cvals - (1.0 - thr)) <= 1e-12, axis=-1)
    assert near.sum() == 0
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("n", [3, 5, 8, 10])
def test_selection_matches_exhaustive_subset_search(n):
    # With distinct values the kept set is the heaviest subset among those of
    # least cardinality whose mass exceeds thr (keep blocks until the kept mass
    # exceeds thr, biggest first). Checked by enumerating every subset.
    rng = np.random.default_rng(n)
    for trial in range(6):
        p = rng.dirichlet(np.ones(n) * 0.7)
        thr = float(rng.uniform(0.05, 0.95))
        got = oracle.cdf_mask(oracle.mass_above(p[None, None, :].repeat(n, 1)), thr)[0, 0]
        best = None
        for r in range(1, n + 1):
            cands = [c for c in itertools.combinations(range(n), r) if p[list(c)].sum() > thr]
            if cands:
                best = max(cands, key=lambda c: p[list(c)].sum())
                break
        exp = np.zeros(n, dtype=np.uint8)
        exp[list(best)] = 1
        np.testing.assert_array_equal(got, exp, err_msg=f"p={p} thr={thr}")


def test_selection_hand_worked_rows():
    with open(os.path.join(GOLDEN, "cdf_rows.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        p = np.asarray(c["p"], dtype=np.float64)
        n = p.size
        got = oracle.cdf_mask(oracle.mass_above(np.tile(p, (1, n, 1))), c["thr"])[0, 0]
        np.testing.assert_array_equal(got, c["expected"], err_msg=c["why"])


def test_selection_invariants():
    p = _random_probs(2, 64, 12)
    g = oracle.mass_above(p)
    prev = None
    for thr in [0.0, 0.1, 0.3, 0.5, 0.8, 0.95, 0.999, 1.0, 1.5]:
        m = oracle.cdf_mask(g, thr).astype(bool)
        kept_mass = (p * m).sum(-1)
        if thr < 1.0:
            assert np.all(kept_mass > thr)
            # Minimality: dropping the smallest kept entry leaves mass <= thr.
            smallest = np.where(m, p, np.inf).min(-1)
            assert np.all(kept_mass - smallest <= thr + 1e-15)
        else:
            assert m.all()
        # The row maximum is always kept, so no row is empty.
        am = p.argmax(-1)
        assert np.take_along_axis(m, am[..., None], -1).all()
        if prev is not None:
            assert np.all(prev <= m), "masks must be nested in thr"
        prev = m


def test_selection_is_equivariant_under_key_block_permutation():
    q, k = _rand((2, 640, 16), 13), _rand((2, 640, 16), 14)
    perm = np.random.default_rng(15).permutation(10)
    kb = k.reshape(2, 10, 64, 16)[:, perm].reshape(2, 640, 16)
    m0 = oracle.build_mask(q, k, 64, 0.6)["mask"]
    m1 = oracle.build_mask(q, kb, 64, 0.6)["mask"]
    np.testing.assert_array_equal(m1, m0[:, :, perm])


def test_selection_ignores_row_constant_logit_shift():
    # K -> K + c (one vector c for every token) adds q_a.c to a whole row of the
    # reduced logits, which softmax cancels: the mask cannot change.
    q, k = _rand((2, 640, 16), 16), _rand((2, 640, 16), 17)
    c = _rand((1, 1, 16), 18, 3.0)
    m0 = oracle.build_mask(q, k, 64, 0.5)
    m1 = oracle.build_mask(q, k + c, 64, 0.5)
    np.testing.assert_allclose(m0["a"], m1["a"], atol=1e-9)
    np.testing.assert_array_equal(m0["mask"], m1["mask"])


def test_threshold_direction_matches_table1():
    # Table 1: NABLA(0.7) is 80.13% sparse and NABLA(0.4) 92.5%: a larger thr
    # keeps more blocks. Only the direction is fixed by the paper.
    import synth
    w = synth.get_workload("tiny")
    x = synth.make_inputs(w)
    m7 = oracle.build_mask(x["q"], x["k"], w.N, 0.7)["mask"]
    m4 = oracle.build_mask(x["q"], x["k"], w.N, 0.4)["mask"]
    assert m4.mean() < m7.mean()


def test_invalid_threshold_rejected():
    g = np.zeros((1, 2, 2))
    for bad in [-0.1, float("nan")]:
        with pytest.raises(ValueError):
            oracle.cdf_mask(g, bad)


def test_mask_to_lists_round_trip():
    m = (np.random.default_rng(19).random((3, 12, 12)) < 0.3).astype(np.uint8)
    lists = oracle.mask_to_lists(m)
    back = np.zeros_like(m)
    back2 = np.zeros_like(m)
    for bh in range(3):
        for i in range(12):
            js = lists["kv_idx"][bh, i, : lists["kv_count"][bh, i]]
            assert np.all(np.diff(js) > 0)
            back[bh, i, js] = 1
            is_ = lists["q_idx"][bh, i, : lists["q_count"][bh, i]]
            assert np.all(np.diff(is_) > 0)
            back2[bh, is_, i] = 1
    np.testing.assert_array_equal(back, m)
    np.testing.assert_array_equal(back2, m)
