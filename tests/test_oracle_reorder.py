"""Pins of the oracle's token reordering (section 3.1.1, Figure 3)."""

import numpy as np

import oracle


def test_figure3_example_16x16_patch8():
    # Figure 3: a 16 x 16 latent with patch size 8 becomes four contiguous runs of
    # 64 tokens, one per 8 x 8 patch, patches in row-major order.
    perm = oracle.token_order(1, 16, 16, 8)
    assert perm.shape == (256,)
    for blk, (py0, px0) in enumerate([(0, 0), (0, 8), (8, 0), (8, 8)]):
        run = perm[64 * blk:64 * (blk + 1)]
        ys, xs = run // 16, run % 16
        assert ys.min() == py0 and ys.max() == py0 + 7
        assert xs.min() == px0 and xs.max() == px0 + 7
        # row-major inside the patch
        np.testing.assert_array_equal(run[:8], (py0 * 16 + px0) + np.arange(8))
        np.testing.assert_array_equal(run[8:16], ((py0 + 1) * 16 + px0) + np.arange(8))


def test_time_order_is_kept_and_permutation_is_a_bijection():
    T, Hs, Ws, P = 5, 24, 40, 8
    perm = oracle.token_order(T, Hs, Ws, P)
    assert np.array_equal(np.sort(perm), np.arange(T * Hs * Ws))
    frames = perm // (Hs * Ws)
    assert np.all(np.diff(frames) >= 0)          # frames never go back in time
    per_frame = Hs * Ws
    for t in range(T):
        np.testing.assert_array_equal(frames[t * per_frame:(t + 1) * per_frame], t)


def test_inverse_restores_raster_order():
    x = np.random.default_rng(0).standard_normal((3, 2 * 16 * 24, 5)).astype(np.float32)
    y = oracle.tokens_to_blocks(x, 2, 16, 24, 8)
    np.testing.assert_array_equal(oracle.blocks_to_tokens(y, 2, 16, 24, 8), x)
    assert not np.array_equal(y, x)


def test_patch_size_one_is_identity():
    perm = oracle.token_order(3, 4, 5, 1)
    np.testing.assert_array_equal(perm, np.arange(60))
