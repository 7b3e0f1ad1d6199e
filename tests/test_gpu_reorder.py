"""GPU parity of token reordering (section 3.1.1, Figure 3) against the oracle: bit-exact."""

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def _nb():
    import block_sparse_attention_nabla_amd as nb
    nb.load_library()
    return nb


def _bits(items, S, F, dtype, seed):
    """Random bit patterns (NaNs and all) so that any arithmetic on the data would show."""
    g = torch.Generator().manual_seed(seed)
    words = F * dtype.itemsize // 4
    x = torch.randint(-2**31, 2**31 - 1, (items, S, words), generator=g, dtype=torch.int32)
    return x.view(dtype).reshape(items, S, F)


# (items, T, Hs, Ws, P, F, dtype): several workgroups and ragged tails
# (runs not a multiple of runs per workgroup), P = 1, odd patch counts, rows
# from 16 B to 10 KiB (runs larger than one workgroup's share).
CASES = [
    (2, 3, 16, 24, 8, 64, torch.bfloat16),     # 128 B rows, 8 x 8 patches
    (1, 2, 12, 20, 4, 8, torch.float32),       # 32 B rows, 4 x 4 patches
    (3, 5, 6, 10, 2, 4, torch.int32),          # 16 B rows, ragged everywhere
    (1, 1, 16, 16, 8, 5120, torch.bfloat16),   # hidden-state rows of 10 KiB
    (2, 2, 8, 24, 8, 128, torch.bfloat16),     # one patch row per frame
    (1, 3, 5, 7, 1, 8, torch.int32),           # P = 1: identity
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}x{c[3]}_P{c[4]}_F{c[5]}")
def test_reorder_matches_oracle(case):
    nb = _nb()
    items, T, Hs, Ws, P, F, dtype = case
    S = T * Hs * Ws
    x = _bits(items, S, F, dtype, 11)
    xb = x.view(torch.uint8).reshape(items, S, -1).numpy()
    print(f"reorder case items={items} T={T} Hs={Hs} Ws={Ws} P={P} F={F} {dtype}", flush=True)
    y = nb.nabla_reorder_tokens(x.cuda(), T, Hs, Ws, P)
    torch.cuda.synchronize()
    want = oracle.tokens_to_blocks(xb, T, Hs, Ws, P)
    got = y.cpu().view(torch.uint8).reshape(items, S, -1).numpy()
    np.testing.assert_array_equal(got, want)
    z = nb.nabla_reorder_tokens(y, T, Hs, Ws, P, inverse=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(z.cpu().view(torch.uint8).reshape(items, S, -1).numpy(), xb)
    # The inverse on its own (block order in) against the oracle's inverse.
    yb = torch.from_numpy(want.copy()).view(dtype).reshape(items, S, F)
    w = nb.nabla_reorder_tokens(yb.cuda(), T, Hs, Ws, P, inverse=True)
    np.testing.assert_array_equal(w.cpu().view(torch.uint8).reshape(items, S, -1).numpy(),
                                  oracle.blocks_to_tokens(want, T, Hs, Ws, P))


def test_reorder_figure3_grid():
    # Figure 3's 16 x 16 latent with 8 x 8 patches, tokens carrying their raster index.
    nb = _nb()
    x = torch.arange(256, dtype=torch.int32).repeat_interleave(4).reshape(1, 256, 4)
    y = nb.nabla_reorder_tokens(x.cuda(), 1, 16, 16, 8).cpu()[0, :, 0].numpy()
    np.testing.assert_array_equal(y, oracle.token_order(1, 16, 16, 8))


def test_reorder_empty_and_errors():
    nb = _nb()
    x = torch.empty((1, 0, 64), dtype=torch.bfloat16, device="cuda")
    assert nb.nabla_reorder_tokens(x, 0, 16, 16, 8).shape == x.shape
    bad = torch.zeros((1, 12 * 16, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nb.NablaError):
        nb.nabla_reorder_tokens(bad, 1, 12, 16, 8)     # 12 is not a multiple of 8
    odd = torch.zeros((1, 256, 3), dtype=torch.float32, device="cuda")
    with pytest.raises(nb.NablaError):
        nb.nabla_reorder_tokens(odd, 1, 16, 16, 8)     # 12-byte rows


@pytest.mark.parametrize("layout", ["hidden", "heads"])
def test_reorder_full_size_wan720p(layout):
    # The 720p Wan latent (21 x 48 x 80 tokens, 8 x 8 patches): the hidden states
    # [1, S, 5120] bf16 and the per-head layout [40, S, 128] bf16. Sampled rows
    # against the oracle's permutation, and the round trip everywhere.
    nb = _nb()
    T, Hs, Ws, P = 21, 48, 80, 8
    S = T * Hs * Ws
    shape = (1, S, 5120) if layout == "hidden" else (40, S, 128)
    print(f"reorder full size {layout} {shape}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(5)
    x = torch.randint(-2**15, 2**15 - 1, shape, generator=g, device="cuda",
                      dtype=torch.int16).view(torch.bfloat16)
    y = nb.nabla_reorder_tokens(x, T, Hs, Ws, P)
    z = nb.nabla_reorder_tokens(y, T, Hs, Ws, P, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(z.view(torch.int16), x.view(torch.int16))
    perm = torch.from_numpy(oracle.token_order(T, Hs, Ws, P))
    rng = np.random.default_rng(1)
    pos = torch.from_numpy(rng.choice(S, size=2048, replace=False))
    pos = torch.cat([pos, torch.tensor([0, S - 1])])
    for item in sorted({0, shape[0] - 1}):
        got = y[item, pos.cuda()].view(torch.int16).cpu()
        want = x[item, perm[pos].cuda()].view(torch.int16).cpu()
        assert torch.equal(got, want)
