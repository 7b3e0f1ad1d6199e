"""GPU parity of the variant selectors against the oracle: Top-k blocks (with and
without the STA union) and the static STA mask alone, and attention over their
lists through the same forward kernel."""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (O_MAX_ABS, O_MEAN_ABS, attn_errors, compare_topk_masks, lists_to_mask)

pytestmark = pytest.mark.gpu


def _nb():
    import block_sparse_attention_nabla_amd as nb
    nb.load_library()
    return nb


def _check_lists(out, n_min=1):
    B, H, n = out["kv_count"].shape
    dense = out["dense_mask"].reshape(B * H, n, n)
    np.testing.assert_array_equal(lists_to_mask(out["kv_count"], out["kv_idx"]), dense)
    if "q_count" in out:
        np.testing.assert_array_equal(lists_to_mask(out["q_count"], out["q_idx"]),
                                      np.swapaxes(dense, 1, 2))
    assert (out["kv_count"] >= n_min).all()
    return dense


def _topk_case(q, k, topk, sta=None):
    nb = _nb()
    print(f"[topk] shape={tuple(q.shape)} k={topk} sta={sta}", flush=True)
    out = nb.nabla_build_topk_mask(q.cuda(), k.cuda(), topk, sta, transpose=True, dense=True)
    torch.cuda.synchronize()
    gpu = {key: val.cpu().numpy() for key, val in out.items()}
    n = gpu["kv_count"].shape[-1]
    dense = _check_lists(gpu, n_min=min(topk, n))
    orc = oracle.build_topk_mask(q.float(), k.float(), 64, topk, sta=sta)
    sta_map = None
    if sta is not None:
        sta_map = oracle.sta_mask(sta["T"], sta["Hs"], sta["Ws"], sta["P"], sta["win_t"],
                                  sta["win_h"], sta["win_w"])
    res = compare_topk_masks(dense, orc, topk, sta_map)
    print(f"[topk] {res}", flush=True)
    assert res["unexplained"] == 0, res
    return gpu, out


@pytest.mark.parametrize("topk", [1, 2, 5, 16, 40])
def test_topk_tiny(topk):
    w = synth.get_workload("tiny")
    x = synth.make_inputs(w)
    gpu, _ = _topk_case(x["q"].bfloat16(), x["k"].bfloat16(), topk)
    if topk >= w.n:
        assert gpu["dense_mask"].all()


@pytest.mark.parametrize("topk", [8, 40, 200])
def test_topk_dit_small(topk):
    w = synth.get_workload("dit_small")
    x = synth.make_inputs(w)
    _topk_case(x["q"], x["k"], topk)


def test_topk_with_sta_union():
    w = synth.get_workload("dit_small_sta")
    x = synth.make_inputs(w)
    _topk_case(x["q"], x["k"], 12, w.sta_struct())


@pytest.mark.parametrize("n,BH,topk", [(37, 3, 7), (300, 2, 29), (2, 4, 1)])
def test_topk_ragged_rows(n, BH, topk):
    g = torch.Generator().manual_seed(n)
    q = (torch.randn((1, BH, 64 * n, 64), generator=g) * 2).bfloat16()
    k = (torch.randn((1, BH, 64 * n, 64), generator=g) * 2).bfloat16()
    _topk_case(q, k, topk)


def test_topk_ties_are_kept_together():
    # Key blocks 0..3 duplicated as 4..7: every reduced-map entry has an exact twin,
    # so top-k with odd k keeps the twin of the k-th entry as well.
    g = torch.Generator().manual_seed(9)
    B, H, n = 1, 2, 8
    q = torch.randn((B, H, 64 * n, 64), generator=g).bfloat16()
    k = torch.randn((B, H, 64 * n, 64), generator=g).bfloat16()
    k[:, :, 64 * 4:] = k[:, :, :64 * 4]
    gpu, _ = _topk_case(q, k, 3)
    assert (gpu["kv_count"] == 4).all()


def _sta_only_case(B, H, sta):
    nb = _nb()
    S = sta["T"] * sta["Hs"] * sta["Ws"]
    print(f"[sta] B={B} H={H} S={S} {sta}", flush=True)
    out = nb.nabla_build_sta_mask(B, H, S, sta, "cuda", transpose=True, dense=True)
    torch.cuda.synchronize()
    gpu = {key: val.cpu().numpy() for key, val in out.items()}
    dense = _check_lists(gpu)
    want = oracle.sta_only_mask(B * H, sta["T"], sta["Hs"], sta["Ws"], sta["P"], sta["win_t"],
                                sta["win_h"], sta["win_w"])
    np.testing.assert_array_equal(dense, want)          # integer work: bit-exact
    return out


@pytest.mark.parametrize("sta", [
    dict(T=4, Hs=16, Ws=16, P=8, win_t=3, win_h=8, win_w=16),
    dict(T=11, Hs=32, Ws=32, P=8, win_t=11, win_h=24, win_w=24),
    dict(T=5, Hs=24, Ws=40, P=8, win_t=2, win_h=16, win_w=24),     # even windows: asymmetric
    dict(T=1, Hs=8, Ws=8, P=8, win_t=1, win_h=8, win_w=8),         # n = 1
])
def test_sta_only_exact(sta):
    _sta_only_case(1, 3, sta)


@pytest.mark.parametrize("win", [(18, 40, 40), (18, 24, 24)])
def test_sta_only_720p_table1_windows(win):
    # Table 1's STA rows on the 720p latent grid: exact lists, and the sparsity the
    # oracle's clipped window gives (80.24% and 91.62%).
    sta = dict(T=21, Hs=48, Ws=80, P=8, win_t=win[0], win_h=win[1], win_w=win[2])
    out = _sta_only_case(1, 2, sta)
    n = out["kv_count"].shape[-1]
    sparsity = 1 - int(out["kv_count"].sum()) / (2 * n * n)
    print(f"[sta] 720p {win}: sparsity {sparsity:.4f}", flush=True)
    assert abs(sparsity - {40: 0.8024, 24: 0.9162}[win[1]]) < 5e-4


def test_attention_over_variant_lists():
    # The forward kernel over Top-k lists and over STA-only lists, against the
    # oracle's masked attention on the same masks.
    nb = _nb()
    w = synth.get_workload("dit_small_sta")
    x = synth.make_inputs(w)
    xg = {key: val.cuda() for key, val in x.items()}
    for name in ("topk", "sta"):
        if name == "topk":
            out = nb.nabla_build_topk_mask(xg["q"], xg["k"], 24, dense=True)
        else:
            out = nb.nabla_build_sta_mask(w.B, w.H, w.S, w.sta_struct(), "cuda", dense=True)
        o, lse = nb.nabla_sparse_attn_fwd(xg["q"], xg["k"], xg["v"], out["kv_count"], out["kv_idx"])
        torch.cuda.synchronize()
        mask = out["dense_mask"].cpu().numpy().reshape(w.B * w.H, w.n, w.n)
        blocks = list(range(0, w.B * w.H * w.n, 37))
        ro, rlse = oracle.attn_fwd(x["q"].float(), x["k"].float(), x["v"].float(), mask, w.N,
                                   blocks=blocks)
        of = o.float().cpu().numpy().reshape(w.B * w.H, w.S, w.D)
        sel = ~np.isnan(ro[..., 0])
        e = attn_errors(of[sel], ro[sel])
        dl = float(np.abs(lse.cpu().numpy().reshape(w.B * w.H, w.S)[sel] - rlse[sel]).max())
        print(f"[variants] fwd over {name} lists: blocks={len(blocks)} {e} lse={dl:.2e}", flush=True)
        assert e["max_abs"] <= O_MAX_ABS and e["mean_abs"] <= O_MEAN_ABS, e
        assert dl <= 1e-3


def test_topk_720p_full_size():
    # Top-k at the 720p layer with k = 126 (10% of the 1260 blocks, the same mean
    # density as the CDF rule at 90%): every head on the GPU and by the oracle.
    nb = _nb()
    w = synth.get_workload("wan14b_720p")
    x = synth.make_inputs(w)
    q, k = x["q"].cuda(), x["k"].cuda()
    topk = 126
    out = nb.nabla_build_topk_mask(q, k, topk, dense=True)
    torch.cuda.synchronize()
    cnt = out["kv_count"].cpu().numpy()
    assert (cnt >= topk).all()
    print(f"[topk] 720p k={topk}: rows above k {int((cnt > topk).sum())}, "
          f"sparsity {1 - cnt.sum() / (w.B * w.H * w.n * w.n):.5f}", flush=True)
    dense = out["dense_mask"].reshape(w.B * w.H, w.n, w.n)
    res_all = []
    for bh in range(w.B * w.H):
        orc = oracle.build_topk_mask(x["q"].reshape(-1, w.S, w.D)[bh:bh + 1].float(),
                                     x["k"].reshape(-1, w.S, w.D)[bh:bh + 1].float(), w.N, topk)
        res = compare_topk_masks(dense[bh:bh + 1].cpu().numpy(), orc, topk)
        res_all.append(res)
        assert res["unexplained"] == 0, (bh, res)
    tot = {key: sum(r[key] for r in res_all) for key in res_all[0]}
    print(f"[topk] 720p all {len(res_all)} heads: {tot}", flush=True)


def test_topk_order_below_fp32_resolution_is_exact():
    # Two key blocks whose reduced probabilities differ by ~1e-8 relative (below
    # fp32 resolution); k chosen so that the cut falls between them: only the
    # larger one is kept, as in the oracle.
    from test_gpu_mask import _near_tied_pair
    b = 9
    q, k, p, a = _near_tied_pair(b=b)
    hi, lo = (a, b) if p[0, a] > p[0, b] else (b, a)
    topk = int((p[0] > p[0, hi]).sum()) + 1
    gpu, _ = _topk_case(q, k, topk)
    dense = gpu["dense_mask"].reshape(32, 32)
    assert dense[0, hi] == 1 and dense[0, lo] == 0
