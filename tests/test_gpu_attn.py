"""GPU parity of block-sparse attention (forward and backward) against the oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (grad_ok, LSE_MAX_ABS, O_MAX_ABS, O_MEAN_ABS, attn_errors,
                    grad_errors, lists_to_mask)

pytestmark = pytest.mark.gpu


def _nb():
    import block_sparse_attention_nabla_amd as nb
    nb.load_library()
    return nb


def _lists_from_mask(mask: np.ndarray, B, H):
    lists = oracle.mask_to_lists(mask)
    n = mask.shape[-1]
    out = {}
    for key in ("kv_count", "q_count"):
        out[key] = torch.from_numpy(lists[key].reshape(B, H, n)).cuda()
    for key in ("kv_idx", "q_idx"):
        out[key] = torch.from_numpy(lists[key].reshape(B, H, n, n)).cuda()
    return out


def _rand(B, H, S, D, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return [(torch.randn((B, H, S, D), generator=g) * scale).bfloat16() for _ in range(4)]


def _random_mask(BH, n, seed, p):
    rng = np.random.default_rng(seed)
    m = (rng.random((BH, n, n)) < p).astype(np.uint8)
    m[:, np.arange(n), rng.integers(0, n, n)] = 1  # every row keeps something
    return m


def _fwd_check(q, k, v, lists, mask, scale=None, tag="", out_dtype=torch.bfloat16):
    nb = _nb()
    B, H, S, D = q.shape
    print(f"[fwd] {tag} shape={tuple(q.shape)} kept={int(mask.sum())} out={out_dtype}", flush=True)
    o, lse = nb.nabla_sparse_attn_fwd(q.cuda(), k.cuda(), v.cuda(), lists["kv_count"], lists["kv_idx"],
                                      softmax_scale=scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ro, rlse = oracle.attn_fwd(q.float(), k.float(), v.float(), mask, 64, scale=scale)
    e = attn_errors(o.float().cpu().numpy().reshape(B * H, S, D), ro)
    dl = np.abs(lse.cpu().numpy().reshape(B * H, S) - rlse)
    print(f"[fwd] {tag} {e} lse_max_abs={dl.max():.2e}", flush=True)
    assert e["max_abs"] <= O_MAX_ABS and e["mean_abs"] <= O_MEAN_ABS, e
    assert dl.max() <= LSE_MAX_ABS
    return o, lse


@pytest.mark.parametrize("thr", [0.2, 0.5, 0.9, 1.0])
def test_fwd_tiny_with_gpu_mask(thr):
    nb = _nb()
    w = synth.get_workload("tiny")
    x = synth.make_inputs(w)
    q, k, v = (x[key].bfloat16() for key in ("q", "k", "v"))
    lists = nb.nabla_build_mask(q.cuda(), k.cuda(), thr, transpose=True)
    torch.cuda.synchronize()
    mask = lists_to_mask(lists["kv_count"].cpu().numpy(), lists["kv_idx"].cpu().numpy())
    # The tiny workload is fp32: its output is stored as fp32 (|O| reaches ~9 here,
    # where bf16 storage alone would be off by up to 0.03).
    _fwd_check(q, k, v, lists, mask, tag=f"tiny thr={thr}", out_dtype=torch.float32)


@pytest.mark.parametrize("name", ["dit_small", "dit_small_sta"])
def test_fwd_dit_small_with_gpu_mask(name):
    nb = _nb()
    w = synth.get_workload(name)
    x = synth.make_inputs(w)
    thr = w.thresholds()[0]
    lists = nb.nabla_build_mask(x["q"].cuda(), x["k"].cuda(), thr, w.sta_struct())
    torch.cuda.synchronize()
    mask = lists_to_mask(lists["kv_count"].cpu().numpy(), lists["kv_idx"].cpu().numpy())
    _fwd_check(x["q"], x["k"], x["v"], lists, mask, tag=name)


@pytest.mark.parametrize("B,H,n,D,p", [(1, 2, 9, 64, 0.4), (2, 1, 33, 128, 0.3), (1, 1, 1, 128, 1.0),
                                       (1, 3, 70, 64, 0.15)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_fwd_random_masks(B, H, n, D, p, out_dtype):
    q, k, v, _ = _rand(B, H, 64 * n, D, seed=n + D, scale=1.5)
    mask = _random_mask(B * H, n, n, p)
    _fwd_check(q, k, v, _lists_from_mask(mask, B, H), mask, tag="random", out_dtype=out_dtype)


@pytest.mark.parametrize("D", [64, 128])
def test_fwd_running_maximum_growth(D):
    """Key blocks scaled so that each row's maximum logit moves by different amounts from
    block to block (about 4.3 log2 units per unit of scale step): steps where it grows by
    more than 2^8 (the output is rescaled), steps where probabilities against the running
    maximum exceed 2^7 without such growth (the block maximum is formed and no rescale
    follows), and steps where it falls. Compared with the oracle, unpaired and paired, and
    the two launches bitwise."""
    nb = _nb()
    n, H = 16, 2
    S = 64 * n
    scales = [0.5, 0.6, 1.5, 2.0, 4.5, 4.6, 5.8, 8.5, 8.0, 9.5, 3.0, 9.6, 11.0, 1.0, 12.5, 12.6]
    g = torch.Generator().manual_seed(41 + D)
    q = torch.randn((1, H, S, D), generator=g)
    k = torch.randn((1, H, S, D), generator=g) * torch.tensor(scales).repeat_interleave(64).view(1, 1, S, 1)
    v = torch.randn((1, H, S, D), generator=g)
    q, k, v = (t.bfloat16() for t in (q, k, v))
    mask = np.ones((H, n, n), dtype=np.uint8)
    mask[1] = _random_mask(1, n, 5, 0.6)[0]
    lists = _lists_from_mask(mask, 1, H)
    o, lse = _fwd_check(q, k, v, lists, mask, tag=f"growing maxima D={D}", out_dtype=torch.float32)
    o2, lse2 = nb.nabla_sparse_attn_fwd(q.cuda(), k.cuda(), v.cuda(), lists["kv_count"], lists["kv_idx"],
                                        out_dtype=torch.float32, frame_blocks=4)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int32), o2.view(torch.int32))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))


@pytest.mark.parametrize("D", [64, 128])
def test_fwd_constant_values_are_reproduced(D):
    """The weights of each softmax row of eq. (4) (section 2.2) sum to one, so values that
    are the same for every token come out unchanged: O[s, d] = c[d] for every row with a
    kept block. The kernel divides by the sum of the bf16 weights that actually entered the
    PV product, so only fp32 accumulation rounding remains (a division by the fp32 sum of
    the unrounded weights would leave the bf16 rounding of the weights, up to 2^-8 of c).
    Keys scaled as in the running-maximum test, so rescales of the output and the lazy
    block maximum are exercised; unpaired and paired launches."""
    nb = _nb()
    n, H = 16, 2
    S = 64 * n
    scales = [0.5, 0.6, 1.5, 2.0, 4.5, 4.6, 5.8, 8.5, 8.0, 9.5, 3.0, 9.6, 11.0, 1.0, 12.5, 12.6]
    g = torch.Generator().manual_seed(77 + D)
    q = torch.randn((1, H, S, D), generator=g).bfloat16()
    k = (torch.randn((1, H, S, D), generator=g)
         * torch.tensor(scales).repeat_interleave(64).view(1, 1, S, 1)).bfloat16()
    c = (torch.randn((1, H, 1, D), generator=g) * 3.0).bfloat16()
    v = c.expand(1, H, S, D).contiguous()
    mask = np.ones((H, n, n), dtype=np.uint8)
    mask[1] = _random_mask(1, n, 9, 0.5)[0]
    lists = _lists_from_mask(mask, 1, H)
    want = c.float().expand(1, H, S, D)
    for F in (0, 4):
        o, _ = nb.nabla_sparse_attn_fwd(q.cuda(), k.cuda(), v.cuda(), lists["kv_count"], lists["kv_idx"],
                                        out_dtype=torch.float32, frame_blocks=F)
        torch.cuda.synchronize()
        rel = ((o.cpu() - want).abs() / want.abs().clamp_min(1e-30)).max().item()
        print(f"[fwd] constant values D={D} F={F}: max relative deviation {rel:.2e}", flush=True)
        assert rel <= 3e-5, rel


def test_fwd_keep_all_equals_dense_and_custom_scale():
    q, k, v, _ = _rand(1, 2, 64 * 12, 128, seed=11, scale=2.0)
    mask = np.ones((2, 12, 12), dtype=np.uint8)
    _fwd_check(q, k, v, _lists_from_mask(mask, 1, 2), mask, scale=0.05, tag="dense scale=0.05")


def test_fwd_empty_rows_give_zero_and_minus_inf():
    nb = _nb()
    q, k, v, _ = _rand(1, 1, 64 * 4, 64, seed=12)
    mask = np.eye(4, dtype=np.uint8)[None]
    lists = _lists_from_mask(mask, 1, 1)
    lists["kv_count"][0, 0, 2] = 0
    o, lse = nb.nabla_sparse_attn_fwd(q.cuda(), k.cuda(), v.cuda(), lists["kv_count"], lists["kv_idx"])
    torch.cuda.synchronize()
    assert torch.all(o[0, 0, 128:192] == 0)
    assert torch.all(torch.isneginf(lse[0, 0, 128:192]))
    mask[0, 2, 2] = 0
    ro, _ = oracle.attn_fwd(q.float(), k.float(), v.float(), np.maximum(mask, np.eye(4, dtype=np.uint8)), 64)
    e = attn_errors(o.float().cpu().numpy()[0, 0, :128], ro[0, :128])
    assert e["max_abs"] <= O_MAX_ABS


def test_fwd_values_in_dropped_blocks_are_never_read():
    nb = _nb()
    q, k, v, _ = _rand(1, 1, 64 * 6, 128, seed=13)
    mask = np.zeros((1, 6, 6), dtype=np.uint8)
    mask[0, :, 1] = 1
    mask[0, :, 4] = 1
    lists = _lists_from_mask(mask, 1, 1)
    o1, _ = nb.nabla_sparse_attn_fwd(q.cuda(), k.cuda(), v.cuda(), lists["kv_count"], lists["kv_idx"])
    v2 = v.clone()
    v2[:, :, 128:256] = float("nan")
    o2, _ = nb.nabla_sparse_attn_fwd(q.cuda(), k.cuda(), v2.cuda(), lists["kv_count"], lists["kv_idx"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_fwd_is_deterministic():
    nb = _nb()
    q, k, v, _ = _rand(1, 4, 64 * 40, 128, seed=14)
    mask = _random_mask(4, 40, 15, 0.3)
    lists = _lists_from_mask(mask, 1, 4)
    a = nb.nabla_sparse_attn_fwd(q.cuda(), k.cuda(), v.cuda(), lists["kv_count"], lists["kv_idx"])
    b = nb.nabla_sparse_attn_fwd(q.cuda(), k.cuda(), v.cuda(), lists["kv_count"], lists["kv_idx"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# Paired forward (frame_blocks = F): query blocks i and i + F share one workgroup.
# Every block still visits its own kept blocks in ascending order with the same
# arithmetic, so the outputs equal the unpaired kernel's bit for bit; the paired
# output is also checked against the oracle element by element.
@pytest.mark.parametrize("name,F", [("tiny", 4), ("tiny", 1), ("dit_small", 16), ("dit_small_sta", 16)])
def test_fwd_frame_pairs(name, F):
    nb = _nb()
    w = synth.get_workload(name)
    x = synth.make_inputs(w)
    q, k, v = (x[key].bfloat16().cuda() for key in ("q", "k", "v"))
    assert F in (1, (w.Hs // w.P) * (w.Ws // w.P))
    thr = 0.5 if name == "tiny" else w.thr_for(0.80)
    lists = nb.nabla_build_mask(q, k, thr, w.sta_struct(), dense=True)
    print(f"[fwd-pair] {name} F={F} n={w.n} D={w.D}", flush=True)
    mask = lists["dense_mask"].reshape(w.B * w.H, w.n, w.n).cpu().numpy()
    ro, rlse = oracle.attn_fwd(x["q"].bfloat16().float(), x["k"].bfloat16().float(),
                               x["v"].bfloat16().float(), mask, w.N)
    outs = {}
    for out_dtype in (torch.float32, torch.bfloat16):
        o0, l0 = nb.nabla_sparse_attn_fwd(q, k, v, lists["kv_count"], lists["kv_idx"], out_dtype=out_dtype)
        o1, l1 = nb.nabla_sparse_attn_fwd(q, k, v, lists["kv_count"], lists["kv_idx"], out_dtype=out_dtype,
                                          frame_blocks=F)
        torch.cuda.synchronize()
        outs[out_dtype] = o1
        assert torch.equal(o0.view(torch.int16) if out_dtype == torch.bfloat16 else o0.view(torch.int32),
                           o1.view(torch.int16) if out_dtype == torch.bfloat16 else o1.view(torch.int32))
        assert torch.equal(l0.view(torch.int32), l1.view(torch.int32))
        dd = float((o1.float() - o0.float()).abs().max())
        dl = float(np.abs(l1.cpu().numpy().reshape(w.B * w.H, w.S) - rlse).max())
        print(f"[fwd-pair] {out_dtype}: lse vs oracle {dl:.2e}; vs unpaired max {dd:.2e}", flush=True)
        assert dl <= LSE_MAX_ABS and dd <= O_MAX_ABS
    # The fp32 output against the oracle (the tiny workload's |O| reaches 9, where
    # bf16 rounding alone is 0.03); the bf16 output is that value rounded.
    got = outs[torch.float32].cpu().numpy().reshape(w.B * w.H, w.S, w.D)
    e = attn_errors(got, ro)
    print(f"[fwd-pair] fp32 output vs oracle {e}", flush=True)
    assert e["max_abs"] <= O_MAX_ABS and e["mean_abs"] <= O_MEAN_ABS, e
    o32 = outs[torch.float32]
    assert ((outs[torch.bfloat16].float() - o32).abs() <= 2.0 ** -8 * o32.abs() + 1e-6).all()


@pytest.mark.parametrize("D", [64, 128])
def test_fwd_frame_pairs_edge_lists(D):
    # Empty, single and identical lists, odd frame count (last frame unpaired),
    # one partner empty: against the unpaired kernel (bitwise) and the oracle.
    nb = _nb()
    B, H, T, F = 1, 3, 5, 4
    n = T * F
    q, k, v, _ = _rand(B, H, 64 * n, D, seed=21)
    mask = _random_mask(B * H, n, 22, 0.25)
    mask[0, 3] = 0                      # empty row, partner (7) non-empty
    mask[1, 2] = mask[1, 6]             # identical partner lists
    mask[2, 16:20] = 0                  # the unpaired last frame: empty rows
    mask[2, 16, 3] = 1
    mask[0, 9] = 0
    mask[0, 13] = 0                     # both partners empty
    mask[1, 0] = 0
    mask[1, 0, 19] = 1                  # a single kept block, the last one
    lists = _lists_from_mask(mask, B, H)
    o0, l0 = nb.nabla_sparse_attn_fwd(q.cuda(), k.cuda(), v.cuda(), lists["kv_count"], lists["kv_idx"],
                                      out_dtype=torch.float32)
    o1, l1 = nb.nabla_sparse_attn_fwd(q.cuda(), k.cuda(), v.cuda(), lists["kv_count"], lists["kv_idx"],
                                      out_dtype=torch.float32, frame_blocks=F)
    torch.cuda.synchronize()
    assert torch.equal(o0.view(torch.int32), o1.view(torch.int32))
    assert torch.equal(l0.view(torch.int32), l1.view(torch.int32))
    keep = mask.copy()
    ro, rlse = oracle.attn_fwd(q.float(), k.float(), v.float(), keep, 64)
    got = o1.cpu().numpy().reshape(B * H, 64 * n, D)
    rows = keep.sum(axis=-1).repeat(64, axis=-1) > 0
    e = attn_errors(got[rows], ro[rows])
    assert e["max_abs"] <= O_MAX_ABS and e["mean_abs"] <= O_MEAN_ABS, e
    dl = float(np.abs(l1.cpu().numpy().reshape(B * H, 64 * n)[rows] - rlse[rows]).max())
    assert dl <= LSE_MAX_ABS, dl
    assert (got[~rows] == 0).all()
    assert torch.isneginf(l1.cpu().reshape(B * H, 64 * n)[torch.from_numpy(~rows)]).all()


# ------------------------------------------------------------------ backward
def _bwd_check(q, k, v, do, lists, mask, tag="", q_blocks=None, kv_blocks=None,
               o_dtype=torch.bfloat16):
    nb = _nb()
    B, H, S, D = q.shape
    print(f"[bwd] {tag} shape={tuple(q.shape)} kept={int(mask.sum())} o={o_dtype}", flush=True)
    qg, kg, vg, dog = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = nb.nabla_sparse_attn_fwd(qg, kg, vg, lists["kv_count"], lists["kv_idx"], out_dtype=o_dtype)
    dq, dk, dv = nb.nabla_sparse_attn_bwd(qg, kg, vg, o, dog, lse, lists["kv_count"], lists["kv_idx"],
                                          lists["q_count"], lists["q_idx"])
    torch.cuda.synchronize()
    rdq, rdk, rdv = oracle.attn_bwd(q.float(), k.float(), v.float(), do.float(), mask, 64,
                                    q_blocks=q_blocks, kv_blocks=kv_blocks)
    res = {}
    for name, g, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        gg = g.float().cpu().numpy().reshape(B * H, S, D)
        sel = ~np.isnan(r[..., 0])
        res[name] = grad_errors(gg[sel], r[sel])
    print(f"[bwd] {tag} {res}", flush=True)
    for name, e in res.items():
        assert grad_ok(e), (name, e)
    return dq, dk, dv


@pytest.mark.parametrize("D", [64, 128])
def test_bwd_constant_values_give_zero_dq_dk(D):
    """Gradients of eq. (4) (section 2.2) when the values are the same for every token: the
    output does not depend on the attention weights, so dQ = dK = 0 exactly, while
    dV_j = sum_i P_ij dO_i. Here dP_ij = dO_i . c is the same for every key and equals
    Delta_i = dO_i . O_i, so the kernels' dP - Delta (the dP products accumulated from
    -Delta) must cancel to fp32 rounding. dQ and dK are checked against a bound far below
    their size with non-constant values; dV against the oracle."""
    nb = _nb()
    n, H = 12, 2
    S = 64 * n
    g = torch.Generator().manual_seed(91 + D)
    q = (torch.randn((1, H, S, D), generator=g) * 1.5).bfloat16()
    k = (torch.randn((1, H, S, D), generator=g) * 1.5).bfloat16()
    c = (torch.randn((1, H, 1, D), generator=g) * 2.0).bfloat16()
    v = c.expand(1, H, S, D).contiguous()
    do = torch.randn((1, H, S, D), generator=g).bfloat16()
    mask = np.ones((H, n, n), dtype=np.uint8)
    mask[1] = _random_mask(1, n, 13, 0.5)[0]
    lists = _lists_from_mask(mask, 1, H)
    qg, kg, vg, dog = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = nb.nabla_sparse_attn_fwd(qg, kg, vg, lists["kv_count"], lists["kv_idx"], out_dtype=torch.float32)
    dq, dk, dv = nb.nabla_sparse_attn_bwd(qg, kg, vg, o, dog, lse, lists["kv_count"], lists["kv_idx"],
                                          lists["q_count"], lists["q_idx"])
    torch.cuda.synchronize()
    mdq, mdk = dq.float().abs().max().item(), dk.float().abs().max().item()
    rdq, rdk, rdv = oracle.attn_bwd(q.float(), k.float(), v.float(), do.float(), mask, 64)
    e = grad_errors(dv.float().cpu().numpy().reshape(H, S, D), rdv)
    print(f"[bwd] constant values D={D}: max|dQ| {mdq:.2e} max|dK| {mdk:.2e} "
          f"(oracle {np.abs(rdq).max():.1e}, {np.abs(rdk).max():.1e}); dV {e}", flush=True)
    assert mdq <= 2e-3 and mdk <= 2e-3, (mdq, mdk)
    assert grad_ok(e), e


@pytest.mark.parametrize("thr", [0.5, 1.0])
def test_bwd_tiny_with_gpu_mask(thr):
    nb = _nb()
    w = synth.get_workload("tiny")
    x = synth.make_inputs(w)
    q, k, v = (x[key].bfloat16() for key in ("q", "k", "v"))
    do = synth.make_dout(w).bfloat16()
    lists = nb.nabla_build_mask(q.cuda(), k.cuda(), thr, transpose=True)
    torch.cuda.synchronize()
    mask = lists_to_mask(lists["kv_count"].cpu().numpy(), lists["kv_idx"].cpu().numpy())
    _bwd_check(q, k, v, do, lists, mask, tag=f"tiny thr={thr}", o_dtype=torch.float32)


# D = 128 also with a single block, very sparse lists (empty and one-entry key lists) and dense
# lists (long query loops of both parities), the shapes of the four-wave dK/dV kernel's branches.
@pytest.mark.parametrize("B,H,n,D,p", [(1, 2, 9, 64, 0.4), (2, 1, 21, 128, 0.3), (1, 1, 1, 64, 1.0),
                                       (1, 1, 1, 128, 1.0), (1, 2, 40, 128, 0.04),
                                       (1, 1, 33, 128, 0.9)])
def test_bwd_random_masks(B, H, n, D, p):
    q, k, v, do = _rand(B, H, 64 * n, D, seed=100 + n + D)
    mask = _random_mask(B * H, n, 200 + n, p)
    _bwd_check(q, k, v, do, _lists_from_mask(mask, B, H), mask, tag="random")


def test_bwd_dit_small_sampled():
    # Full dit_small shape with the GPU mask; oracle gradients on sampled blocks.
    nb = _nb()
    w = synth.get_workload("dit_small")
    x = synth.make_inputs(w)
    do = synth.make_dout(w)
    lists = nb.nabla_build_mask(x["q"].cuda(), x["k"].cuda(), w.thresholds()[0], transpose=True)
    torch.cuda.synchronize()
    mask = lists_to_mask(lists["kv_count"].cpu().numpy(), lists["kv_idx"].cpu().numpy())
    rng = np.random.default_rng(0)
    blocks = sorted(rng.choice(w.B * w.H * w.n, 24, replace=False).tolist())
    _bwd_check(x["q"], x["k"], x["v"], do, lists, mask, tag="dit_small", q_blocks=blocks,
               kv_blocks=blocks)


def test_bwd_is_deterministic():
    nb = _nb()
    q, k, v, do = _rand(1, 2, 64 * 30, 128, seed=300)
    mask = _random_mask(2, 30, 301, 0.3)
    lists = _lists_from_mask(mask, 1, 2)
    qg, kg, vg, dog = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = nb.nabla_sparse_attn_fwd(qg, kg, vg, lists["kv_count"], lists["kv_idx"])
    a = nb.nabla_sparse_attn_bwd(qg, kg, vg, o, dog, lse, lists["kv_count"], lists["kv_idx"],
                                 lists["q_count"], lists["q_idx"])
    b = nb.nabla_sparse_attn_bwd(qg, kg, vg, o, dog, lse, lists["kv_count"], lists["kv_idx"],
                                 lists["q_count"], lists["q_idx"])
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
