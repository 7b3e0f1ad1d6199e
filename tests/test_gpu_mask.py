"""GPU parity of the mask stage: nabla_build_mask against the CPU oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import compare_masks, lists_to_mask

pytestmark = pytest.mark.gpu


def _nb():
    import block_sparse_attention_nabla_amd as nb
    nb.load_library()
    return nb


def _run(q_bf16, k_bf16, thr, sta=None):
    """GPU mask (dense + lists + transpose) and the oracle on the same bf16 values."""
    nb = _nb()
    print(f"[mask] shape={tuple(q_bf16.shape)} thr={thr} sta={sta}", flush=True)
    qg, kg = q_bf16.cuda(), k_bf16.cuda()
    out = nb.nabla_build_mask(qg, kg, thr, sta, transpose=True, dense=True)
    torch.cuda.synchronize()
    gpu = {key: val.cpu().numpy() for key, val in out.items()}
    orc = oracle.build_mask(q_bf16.float(), k_bf16.float(), 64, thr, sta=sta)
    return gpu, orc


def _check_lists(gpu):
    B, H, n = gpu["kv_count"].shape
    dense = gpu["dense_mask"].reshape(B * H, n, n)
    m = lists_to_mask(gpu["kv_count"], gpu["kv_idx"])
    np.testing.assert_array_equal(m, dense)  # lists are exactly the dense mask, ascending
    mt = lists_to_mask(gpu["q_count"], gpu["q_idx"])
    np.testing.assert_array_equal(mt, np.swapaxes(dense, 1, 2))  # exact transpose
    assert (gpu["kv_count"] >= 1).all(), "every row keeps its largest entry"
    return dense


def _assert_parity(gpu, orc, thr, sta_map=None):
    dense = _check_lists(gpu)
    res = compare_masks(dense, orc, thr, sta_map)
    print(f"[mask] {res}", flush=True)
    assert res["unexplained"] == 0, res
    return res


@pytest.mark.parametrize("thr", [0.2, 0.5, 0.9, 1.0])
def test_mask_tiny_threshold_sweep(thr):
    w = synth.get_workload("tiny")
    x = synth.make_inputs(w)
    gpu, orc = _run(x["q"].bfloat16(), x["k"].bfloat16(), thr)
    _assert_parity(gpu, orc, thr)
    if thr >= 1.0:
        assert gpu["dense_mask"].all()


@pytest.mark.parametrize("name", ["dit_small", "dit_small_std3"])
def test_mask_dit_small(name):
    w = synth.get_workload(name)
    x = synth.make_inputs(w)
    thr = w.thresholds()[0]
    gpu, orc = _run(x["q"], x["k"], thr)
    res = _assert_parity(gpu, orc, thr)
    sparsity = 1.0 - res["kept_gpu"] / res["blocks"]
    assert abs(sparsity - 0.80) < 0.01


def test_mask_with_sta_union():
    w = synth.get_workload("dit_small_sta")
    x = synth.make_inputs(w)
    thr = w.thresholds()[0]
    sta = w.sta_struct()
    gpu, orc = _run(x["q"], x["k"], thr, sta)
    sta_map = oracle.sta_mask(**{k: sta[k] for k in ("T", "Hs", "Ws", "P", "win_t", "win_h", "win_w")})
    _assert_parity(gpu, orc, thr, sta_map)
    dense = gpu["dense_mask"].reshape(-1, w.n, w.n).astype(bool)
    assert np.all(dense[:, sta_map.astype(bool)])  # the union contains the STA window
    counts = gpu["kv_count"].reshape(-1)
    assert counts.min() >= 24 and counts.max() <= w.n


def _random_inputs(B, H, S, D, seed, scale=1.0, smooth=True):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, H, S, D), generator=g) * scale
    k = torch.randn((B, H, S, D), generator=g) * scale
    if smooth:  # correlate the tokens of each block a little
        base = torch.randn((B, H, S // 64, 1, D), generator=g) * scale
        q = (q.reshape(B, H, S // 64, 64, D) + base).reshape(B, H, S, D)
        k = (k.reshape(B, H, S // 64, 64, D) + base).reshape(B, H, S, D)
    return q.bfloat16(), k.bfloat16()


@pytest.mark.parametrize("B,H,n,D", [(2, 3, 37, 64), (1, 2, 300, 128), (1, 1, 1, 128), (1, 1, 2, 64),
                                     (1, 2, 257, 128)])
def test_mask_ragged_shapes(B, H, n, D):
    # n not a multiple of 32 / 64 / 256 exercises every tail of the kernels.
    q, k = _random_inputs(B, H, 64 * n, D, seed=n * 7 + D)
    for thr in (0.3, 0.75):
        gpu, orc = _run(q, k, thr)
        _assert_parity(gpu, orc, thr)


@pytest.mark.parametrize("n", [512, 513, 1024, 1025, 1280, 1281, 2048, 2049, 2100])
def test_mask_row_length_kernel_boundaries(n):
    # Rows of up to 2048 blocks run one wave per row with 8, 16, 20 or 32 values per
    # lane in registers; longer rows keep the row in LDS. Both sides of every
    # boundary.
    q, k = _random_inputs(1, 1, 64 * n, 64, seed=n)
    for thr in (0.4,):
        gpu, orc = _run(q, k, thr)
        _assert_parity(gpu, orc, thr)


def test_mask_threshold_zero_keeps_row_maximum_only():
    q, k = _random_inputs(1, 2, 64 * 40, 128, seed=3)
    gpu, orc = _run(q, k, 0.0)
    _assert_parity(gpu, orc, 0.0)
    # Without exact ties the argmax is the only block with G = 0.
    assert (gpu["kv_count"] == 1).all()
    am = orc["a"].argmax(-1)
    np.testing.assert_array_equal(gpu["kv_idx"].reshape(2, 40, 40)[:, :, 0], am)


def test_mask_keep_all_above_one():
    q, k = _random_inputs(1, 2, 64 * 20, 64, seed=4)
    for thr in (1.0, 3.5):
        gpu, _ = _run(q, k, thr)
        assert gpu["dense_mask"].all()
        assert (gpu["kv_count"] == 20).all()


def test_mask_exact_ties_are_kept_together():
    # Identical key blocks give exactly tied reduced probabilities: the tie group
    # is kept or dropped as a whole on both sides.
    B, H, n, D = 1, 1, 16, 64
    q, k = _random_inputs(B, H, 64 * n, D, seed=5)
    k = k.reshape(B, H, n, 64, D)
    k[:, :, 8:] = k[:, :, :8].clone()
    k = k.reshape(B, H, 64 * n, D).contiguous()
    for thr in (0.2, 0.5, 0.8):
        gpu, orc = _run(q, k, thr)
        res = _assert_parity(gpu, orc, thr)
        dense = gpu["dense_mask"].reshape(n, n)
        np.testing.assert_array_equal(dense[:, :8], dense[:, 8:])


@pytest.mark.parametrize("groups", [(100, 200), (300,)])
def test_mask_large_tie_groups(groups):
    # Tie groups larger than a wave (64 entries share every bit of the probability):
    # the selection cannot finish early and runs all four radix passes.
    B, H, D = 1, 2, 64
    n = sum(groups)
    q, k = _random_inputs(B, H, 64 * n, D, seed=11)
    k = k.reshape(B, H, n, 64, D)
    start = 0
    for g_i, size in enumerate(groups):
        k[:, :, start:start + size] = k[:, :, start:start + 1].clone()
        start += size
    k = k.reshape(B, H, 64 * n, D).contiguous()
    for thr in (0.3, 0.7, 0.99):
        gpu, orc = _run(q, k, thr)
        _assert_parity(gpu, orc, thr)
        dense = gpu["dense_mask"].reshape(B * H, n, n)
        start = 0
        for size in groups:  # every group is kept or dropped whole
            blk = dense[:, :, start:start + size]
            assert (blk.min(axis=-1) == blk.max(axis=-1)).all()
            start += size
        if len(groups) == 1:
            assert dense.all()  # one tie group: every entry has nothing strictly above it


def test_mask_is_deterministic():
    nb = _nb()
    q, k = _random_inputs(1, 4, 64 * 150, 128, seed=6)
    qg, kg = q.cuda(), k.cuda()
    a = nb.nabla_build_mask(qg, kg, 0.6, transpose=True, dense=True)
    b = nb.nabla_build_mask(qg, kg, 0.6, transpose=True, dense=True)
    torch.cuda.synchronize()
    for key in ("kv_count", "dense_mask", "q_count"):
        assert torch.equal(a[key], b[key])


def test_mask_row_constant_key_shift_invariance():
    # K + c for one vector c shifts each reduced-logit row by a constant: the
    # GPU mask must not change beyond the parity band.
    q, k = _random_inputs(1, 2, 64 * 48, 64, seed=7)
    c = torch.randn((1, 1, 1, 64), generator=torch.Generator().manual_seed(8)).bfloat16()
    k2 = (k.float() + c.float()).bfloat16()
    g1, orc1 = _run(q, k, 0.5)
    g2, orc2 = _run(q, k2, 0.5)
    r1 = compare_masks(g2["dense_mask"].reshape(orc1["mask"].shape), orc2, 0.5)
    assert r1["unexplained"] == 0, r1


def _near_tied_pair(seed=21, n=32, D=64, b=9):
    """Key block b = key block a (a = row 0's second-largest block) with one bf16
    element nudged by one unit in the last place (the smallest element of the
    feature where row 0's pooled query is smallest): the two reduced probabilities of row 0 differ by
    ~1e-8 relative, below what fp32 logits resolve. Returns bf16 q, k, the
    oracle's fp64 reduced map and a."""
    g = torch.Generator().manual_seed(seed)
    base = torch.randn((1, 1, n, 1, D), generator=g)
    q = (torch.randn((1, 1, n, 64, D), generator=g) + base).reshape(1, 1, 64 * n, D).bfloat16()
    k = (torch.randn((1, 1, n, 64, D), generator=g) + base).reshape(1, 1, n, 64, D).bfloat16()
    qa = oracle.pool(q.float(), 64)[0]
    p0 = oracle.reduced_map(qa[None], oracle.pool(k.reshape(1, 1, 64 * n, D).float(), 64),
                            1.0 / np.sqrt(D))[0]
    a = int(np.argsort(-p0[0])[1])
    assert a != b
    k[:, :, b] = k[:, :, a]
    d = int(np.argmin(np.abs(qa[0])))
    col = k[0, 0, b, :, d].float().abs()
    r = int(torch.argmin(torch.where(col > 0, col, torch.full_like(col, 1e30))))  # smallest ulp
    bits = k[0, 0, b, r, d].view(torch.int16).item()
    k[0, 0, b, r, d] = torch.tensor([bits + 1], dtype=torch.int16).view(torch.bfloat16)[0]
    k = k.reshape(1, 1, 64 * n, D).contiguous()
    p = oracle.reduced_map(qa[None], oracle.pool(k.float(), 64), 1.0 / np.sqrt(D))[0]
    return q, k, p, a


def test_mask_order_below_fp32_resolution_is_exact():
    # Two probabilities closer than fp32 rounding, with thr placed between their
    # mass-above values (half the larger probability away from each, far outside
    # the 1e-5 band): only the larger one may be kept, as in the oracle.
    b = 9
    q, k, p, a = _near_tied_pair(b=b)
    rel = abs(p[0, a] - p[0, b]) / p[0, a]
    assert 0 < rel < 6e-8, rel
    hi, lo = (a, b) if p[0, a] > p[0, b] else (b, a)
    g_hi = p[0][p[0] > p[0, hi]].sum()
    thr = float(g_hi + 0.5 * p[0, hi])
    assert 0.5 * p[0, hi] > 1e-4
    gpu, orc = _run(q, k, thr)
    res = _assert_parity(gpu, orc, thr)
    dense = gpu["dense_mask"].reshape(32, 32)
    assert orc["mask"].reshape(32, 32)[0, hi] == 1 and orc["mask"].reshape(32, 32)[0, lo] == 0
    assert dense[0, hi] == 1 and dense[0, lo] == 0, res


def test_mask_order_below_fp32_resolution_with_d128_and_long_rows():
    # The same near tie inside long rows (n = 1280 and n = 2100: registers and
    # LDS row variants) at D = 128.
    for n in (1280, 2100):
        b = n - 7
        q, k, p, a = _near_tied_pair(seed=n, n=n, D=128, b=b)
        rel = abs(p[0, a] - p[0, b]) / p[0, a]
        hi, lo = (a, b) if p[0, a] > p[0, b] else (b, a)
        g_hi = p[0][p[0] > p[0, hi]].sum()
        thr = float(g_hi + 0.5 * p[0, hi])
        print(f"[mask] n={n} rel gap {rel:.2e} thr={thr:.6f} half-gap {0.5 * p[0, hi]:.2e}", flush=True)
        assert 0 < rel < 6e-8, rel
        gpu, orc = _run(q, k, thr)
        _assert_parity(gpu, orc, thr)
        dense = gpu["dense_mask"].reshape(n, n)
        assert 0.5 * p[0, hi] > 1e-4
        assert dense[0, hi] == 1 and dense[0, lo] == 0
