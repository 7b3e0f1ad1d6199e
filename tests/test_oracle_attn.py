"""Pins of the oracle's masked attention, forward and backward (eq. (2)-(4))."""

import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def _token_mask(mask, N):
    """Expand a block mask [BH, n, n] to a boolean token mask [BH, S, S] (eq. (4))."""
    m = torch.from_numpy(mask.astype(bool))
    return m.repeat_interleave(N, dim=1).repeat_interleave(N, dim=2)


def _sdpa(q, k, v, mask, N):
    """Library attention in fp64 with the block mask as an explicit boolean mask."""
    tq, tk, tv = (torch.from_numpy(x).double() for x in (q, k, v))
    tm = _token_mask(mask, N) if mask is not None else None
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm)
    logits = tq @ tk.transpose(-1, -2) / math.sqrt(q.shape[-1])
    if tm is not None:
        logits = logits.masked_fill(~tm, float("-inf"))
    return o.numpy(), torch.logsumexp(logits, dim=-1).numpy()


def _random_mask(BH, n, seed, p=0.4):
    m = (np.random.default_rng(seed).random((BH, n, n)) < p).astype(np.uint8)
    m[:, np.arange(n), np.arange(n)] = 1  # every row keeps at least one block
    return m


def test_keep_all_equals_dense_attention():
    q, k, v = _rand((2, 256, 32), 1), _rand((2, 256, 32), 2), _rand((2, 256, 32), 3)
    mask = np.ones((2, 4, 4), dtype=np.uint8)
    o, lse = oracle.attn_fwd(q, k, v, mask, 64)
    ref_o, ref_lse = _sdpa(q, k, v, None, 64)
    np.testing.assert_allclose(o, ref_o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_block_masked_attention_equals_explicit_minus_inf_mask():
    q, k, v = _rand((3, 512, 16), 4, 2.0), _rand((3, 512, 16), 5, 2.0), _rand((3, 512, 16), 6)
    mask = _random_mask(3, 8, 7)
    o, lse = oracle.attn_fwd(q, k, v, mask, 64)
    ref_o, ref_lse = _sdpa(q, k, v, mask, 64)
    np.testing.assert_allclose(o, ref_o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_values_in_dropped_blocks_do_not_matter():
    q, k, v = _rand((2, 512, 16), 8), _rand((2, 512, 16), 9), _rand((2, 512, 16), 10)
    mask = _random_mask(2, 8, 11, 0.3)
    mask[:, :, 3] = 0
    mask[:, 3, 3] = 0
    mask[:, 3, 4] = 1
    o0, _ = oracle.attn_fwd(q, k, v, mask, 64)
    v2, k2 = v.copy(), k.copy()
    v2[:, 3 * 64:4 * 64] = 1e3
    k2[:, 3 * 64:4 * 64] = -7.0
    o1, _ = oracle.attn_fwd(q, k2, v2, mask, 64)
    np.testing.assert_array_equal(o0, o1)


def test_single_kept_block_is_local_attention():
    q, k, v = _rand((1, 256, 16), 12), _rand((1, 256, 16), 13), _rand((1, 256, 16), 14)
    mask = np.eye(4, dtype=np.uint8)[None]
    o, _ = oracle.attn_fwd(q, k, v, mask, 64)
    for i in range(4):
        sl = slice(64 * i, 64 * (i + 1))
        ref, _ = _sdpa(q[:, sl], k[:, sl], v[:, sl], None, 64)
        np.testing.assert_allclose(o[:, sl], ref, rtol=1e-11, atol=1e-12)


def test_block_subset_matches_full_computation():
    q, k, v = _rand((2, 512, 16), 15), _rand((2, 512, 16), 16), _rand((2, 512, 16), 17)
    mask = _random_mask(2, 8, 18)
    o, lse = oracle.attn_fwd(q, k, v, mask, 64)
    blocks = [1, 6, 8 + 3, 15]
    o2, lse2 = oracle.attn_fwd(q, k, v, mask, 64, blocks=blocks)
    for b in blocks:
        bh, i = divmod(b, 8)
        sl = slice(64 * i, 64 * (i + 1))
        np.testing.assert_array_equal(o2[bh, sl], o[bh, sl])
        np.testing.assert_array_equal(lse2[bh, sl], lse[bh, sl])
    assert np.isnan(o2[0, 0]).all()


def test_row_constant_key_shift_leaves_output_unchanged():
    q, k, v = _rand((1, 256, 16), 19), _rand((1, 256, 16), 20), _rand((1, 256, 16), 21)
    c = _rand((1, 1, 16), 22)
    mask = _random_mask(1, 4, 23)
    o0, _ = oracle.attn_fwd(q, k, v, mask, 64)
    # Shift every key by c: each query row's logits move by q.c, which softmax cancels.
    o1, _ = oracle.attn_fwd(q.astype(np.float64).astype(np.float32), (k + c).astype(np.float32), v, mask, 64)
    np.testing.assert_allclose(o0, o1, rtol=1e-5, atol=1e-5)


def _loss(q, k, v, dout, mask, N):
    o, _ = oracle.attn_fwd(q, k, v, mask, N)
    return float((o * dout.astype(np.float64)).sum())


def test_backward_matches_central_finite_differences():
    # Small sizes with N = 4; each perturbed coordinate is an fp32-exact step.
    BH, S, D, N = 1, 16, 4, 4
    q, k, v = _rand((BH, S, D), 24), _rand((BH, S, D), 25), _rand((BH, S, D), 26)
    dout = _rand((BH, S, D), 27)
    mask = _random_mask(BH, S // N, 28, 0.5)
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, mask, N)
    h = 2.0 ** -10
    rng = np.random.default_rng(29)
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = (0, int(rng.integers(S)), int(rng.integers(D)))
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd = (_loss(args_p["q"], args_p["k"], args_p["v"], dout, mask, N)
                  - _loss(args_m["q"], args_m["k"], args_m["v"], dout, mask, N)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def test_backward_matches_library_autograd():
    BH, S, D, N = 2, 256, 16, 64
    q, k, v = _rand((BH, S, D), 30), _rand((BH, S, D), 31), _rand((BH, S, D), 32)
    dout = _rand((BH, S, D), 33)
    mask = _random_mask(BH, S // N, 34)
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, mask, N)
    tq, tk, tv = (torch.from_numpy(x).double().requires_grad_() for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=_token_mask(mask, N))
    o.backward(torch.from_numpy(dout).double())
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-11)


def test_backward_block_subsets_match_full():
    BH, S, D, N = 2, 256, 16, 64
    q, k, v = _rand((BH, S, D), 35), _rand((BH, S, D), 36), _rand((BH, S, D), 37)
    dout = _rand((BH, S, D), 38)
    mask = _random_mask(BH, S // N, 39)
    dq, dk, dv = oracle.attn_bwd(q, k, v, dout, mask, N)
    dq2, dk2, dv2 = oracle.attn_bwd(q, k, v, dout, mask, N, q_blocks=[2, 5], kv_blocks=[0, 7])
    np.testing.assert_array_equal(dq2[0, 128:192], dq[0, 128:192])
    np.testing.assert_array_equal(dq2[1, 64:128], dq[1, 64:128])
    np.testing.assert_allclose(dk2[0, 0:64], dk[0, 0:64], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dv2[1, 192:256], dv[1, 192:256], rtol=1e-13, atol=1e-14)
