"""Checks of the seeded input generator (shapes, determinism, block order)."""

import numpy as np
import torch

import synth


def test_generator_is_deterministic_and_shaped():
    w = synth.get_workload("tiny")
    a = synth.make_inputs(w)
    b = synth.make_inputs(w)
    for key in ("q", "k", "v"):
        assert a[key].shape == (w.B, w.H, w.S, w.D)
        assert a[key].dtype == torch.float32
        assert torch.equal(a[key], b[key])
    c = synth.make_inputs(w, step=1)
    assert not torch.equal(a["q"], c["q"])


def test_head_subset_matches_full_generation():
    w = synth.get_workload("tiny")
    full = synth.make_inputs(w)
    sub = synth.make_inputs(w, heads=range(1, 2))
    assert torch.equal(sub["k"][0], full["k"][0, 1])


def test_block_order_groups_each_tile_of_a_frame():
    # Fractal flattening (section 3.1.1, Figure 3): 16 x 16 frame, 8 x 8 tiles.
    perm = synth.block_order_permutation(2, 16, 16, 8).numpy()
    assert sorted(perm.tolist()) == list(range(512))
    for blk in range(8):
        raster = perm[64 * blk:64 * (blk + 1)]
        t, y, x = raster // 256, (raster // 16) % 16, raster % 16
        assert len(set(t.tolist())) == 1                      # one frame
        assert y.max() - y.min() == 7 and x.max() - x.min() == 7  # one 8x8 tile
        assert t[0] == blk // 4                                 # time order kept
    # Row-major inside the tile.
    np.testing.assert_array_equal(perm[:8], np.arange(8))
    np.testing.assert_array_equal(perm[8:16], np.arange(16, 24))


def test_tokens_of_a_block_share_the_smooth_field():
    # Neighbouring tokens (same block) are more alike than tokens of distant blocks.
    w = synth.get_workload("tiny")
    x = synth.make_inputs(w)["k"][0, 0]
    blocks = x.reshape(w.n, w.N, w.D)
    within = (blocks - blocks.mean(1, keepdim=True)).pow(2).mean()
    across = (blocks.mean(1) - blocks.mean((0, 1))).pow(2).mean()
    assert across > 0.05 * within


def test_gaussian_taps():
    t = synth.gaussian_taps()
    assert t.numel() == 17
    assert abs(float(t.sum()) - 1.0) < 1e-12
    assert torch.equal(t, t.flip(0))


def test_generator_block_order_matches_the_oracle_reordering():
    # The generator emits tokens in block order; its permutation and the oracle's
    # reordering are written independently and must agree (section 3.1.1).
    import oracle
    for T, Hs, Ws, P in ((1, 16, 16, 8), (3, 24, 40, 8), (2, 6, 10, 2)):
        np.testing.assert_array_equal(synth.block_order_permutation(T, Hs, Ws, P).numpy(),
                                      oracle.token_order(T, Hs, Ws, P))
