"""The largest supported row: n = 8192 blocks per head (S = 524,288 tokens).

At this size the oracle's selection (quadratic per row) would take minutes, so the
GPU mask is checked against the CDF rule of section 3.1.2 applied to the oracle's
fp64 reduced map row by row, with G_ij (the mass of the entries strictly larger
than p_ij) formed from a descending sort and its cumulative sum: keep iff
G_ij <= thr. The GPU must agree on every block except those with |G_ij - thr|
<= 1e-5, the band the other parity tests allow. Forward (with and without the
frame hint, bitwise equal) and backward are checked on sampled blocks against the
oracle run on the GPU's own mask."""

import numpy as np
import pytest
import torch

import oracle
from parity import (BAND, grad_ok, LSE_MAX_ABS, O_MAX_ABS, O_MEAN_ABS,
                    attn_errors, grad_errors, lists_to_mask)

pytestmark = pytest.mark.gpu

N_MAX = 8192


def _nb():
    import block_sparse_attention_nabla_amd as nb
    nb.load_library()
    return nb


def _inputs(S, D, seed):
    g = torch.Generator().manual_seed(seed)
    n = S // 64
    base = torch.randn((1, 1, n, 1, D), generator=g)
    q = (torch.randn((1, 1, n, 64, D), generator=g) + base).reshape(1, 1, S, D)
    k = (torch.randn((1, 1, n, 64, D), generator=g) + base).reshape(1, 1, S, D)
    v = torch.randn((1, 1, S, D), generator=g)
    do = torch.randn((1, 1, S, D), generator=g)
    return [t.bfloat16() for t in (q, k, v, do)]


def _check_cdf_rows(p: np.ndarray, keep: np.ndarray, thr: float) -> dict:
    """p [n, n] fp64 reduced map rows, keep [n, n] bool GPU decisions."""
    mism = band = band_mism = 0
    for i in range(p.shape[0]):
        row = p[i]
        desc = -np.sort(-row)                       # descending
        csum = np.concatenate([[0.0], np.cumsum(desc)])
        above = np.searchsorted(-desc, -row, side="left")  # entries strictly larger
        g = csum[above]
        want = g <= thr
        in_band = np.abs(g - thr) <= BAND
        diff = want != keep[i]
        mism += int((diff & ~in_band).sum())
        band += int(in_band.sum())
        band_mism += int((diff & in_band).sum())
    return {"rows": int(p.shape[0]), "unexplained": mism, "band": band, "band_mismatch": band_mism}


def test_max_blocks_mask_forward_backward():
    nb = _nb()
    S, D, thr = 64 * N_MAX, 64, 0.3
    print(f"[max] n={N_MAX} S={S} D={D} thr={thr}", flush=True)
    q, k, v, do = _inputs(S, D, seed=77)
    qg, kg, vg, dog = (t.cuda() for t in (q, k, v, do))
    out = nb.nabla_build_mask(qg, kg, thr, transpose=True, dense=True)
    torch.cuda.synchronize()
    cnt = out["kv_count"].cpu().numpy()
    dense = out["dense_mask"].cpu().numpy().reshape(1, N_MAX, N_MAX)
    print(f"[max] kept {int(cnt.sum())} blocks, per row {cnt.min()}..{cnt.max()}", flush=True)
    # lists are exactly the dense mask (ascending, in range) and its transpose
    np.testing.assert_array_equal(lists_to_mask(cnt, out["kv_idx"].cpu().numpy()), dense)
    np.testing.assert_array_equal(
        lists_to_mask(out["q_count"].cpu().numpy(), out["q_idx"].cpu().numpy()), np.swapaxes(dense, 1, 2))
    # the CDF rule on the oracle's fp64 reduced map
    qa, ka = oracle.pool(q.float(), 64), oracle.pool(k.float(), 64)
    p = oracle.reduced_map(qa, ka, 1.0 / np.sqrt(D))[0]
    res = _check_cdf_rows(p, dense[0].astype(bool), thr)
    print(f"[max] CDF rule check {res}", flush=True)
    assert res["unexplained"] == 0, res
    del p

    # forward: with and without the frame hint (64 blocks per frame), bitwise equal
    o, lse = nb.nabla_sparse_attn_fwd(qg, kg, vg, out["kv_count"], out["kv_idx"], out_dtype=torch.float32)
    o2, lse2 = nb.nabla_sparse_attn_fwd(qg, kg, vg, out["kv_count"], out["kv_idx"], out_dtype=torch.float32,
                                        frame_blocks=64)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int32), o2.view(torch.int32))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
    del o2, lse2
    blocks = [0, int(cnt[0, 0].argmax()), N_MAX // 2 + 3, N_MAX - 1]
    ro, rlse = oracle.attn_fwd(q.float(), k.float(), v.float(), dense, 64, blocks=blocks)
    sel = ~np.isnan(ro[..., 0])
    og = o.cpu().numpy().reshape(1, S, D)
    e = attn_errors(og[sel], ro[sel])
    dl = float(np.abs(lse.cpu().numpy().reshape(1, S)[sel] - rlse[sel]).max())
    print(f"[max] fwd sampled blocks {blocks}: {e} lse {dl:.2e}", flush=True)
    assert e["max_abs"] <= O_MAX_ABS and e["mean_abs"] <= O_MEAN_ABS, e
    assert dl <= LSE_MAX_ABS

    # backward on sampled query and key blocks
    dq, dk, dv = nb.nabla_sparse_attn_bwd(qg, kg, vg, o, dog, lse, out["kv_count"], out["kv_idx"],
                                          out["q_count"], out["q_idx"])
    torch.cuda.synchronize()
    cnt_row = out["kv_count"][0, 0].cpu().numpy()
    qb = sorted({5, N_MAX - 2, int(cnt_row.argmax())})  # includes the longest dQ loop
    qc = out["q_count"][0, 0].cpu().numpy()
    # The key block kept by the fewest and by the most query blocks (the longest dK/dV loop).
    kb = sorted({int(np.argmin(np.where(qc > 0, qc, N_MAX + 1))), 9, int(qc.argmax())})
    print(f"[max] bwd key blocks {kb} with q_count {[int(qc[j]) for j in kb]}", flush=True)
    rdq, rdk, rdv = oracle.attn_bwd(q.float(), k.float(), v.float(), do.float(), dense, 64,
                                    q_blocks=qb, kv_blocks=kb)
    res = {}
    for name, g_, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        gg = g_.float().cpu().numpy().reshape(1, S, D)
        m = ~np.isnan(r[..., 0])
        res[name] = grad_errors(gg[m], r[m])
        assert grad_ok(res[name]), (name, res)
    print(f"[max] bwd sampled {res}", flush=True)


def test_mask_map_in_head_chunks():
    """Two heads at n = 6144: one head's reduced map (151 MB) fills the library's
    256 MiB map region alone, so the mask call computes the logits and the
    selection once per head, each into the same region. Both heads' lists must
    follow the CDF rule on the oracle's fp64 map (outside the 1e-5 band), and equal
    what one-head calls on the same data give."""
    nb = _nb()
    n, D, thr, H = 6144, 64, 0.3, 2
    S = 64 * n
    head_map = n * n * 4
    assert 2 * head_map > (256 << 20) >= head_map  # one head per chunk
    assert nb.nabla_workspace_size(nb.NABLA_OP_MASK, 1, H, S, D) < H * head_map
    per_head = [_inputs(S, D, seed=91 + h) for h in range(H)]
    q = torch.cat([t[0] for t in per_head], dim=1)  # [1, H, S, D]
    k = torch.cat([t[1] for t in per_head], dim=1)
    qg, kg = q.cuda(), k.cuda()
    print(f"[chunks] n={n} H={H} D={D} thr={thr}", flush=True)
    out = nb.nabla_build_mask(qg, kg, thr, transpose=True, dense=True)
    torch.cuda.synchronize()
    cnt = out["kv_count"].cpu().numpy()
    dense = out["dense_mask"].cpu().numpy().reshape(H, n, n)
    np.testing.assert_array_equal(lists_to_mask(cnt, out["kv_idx"].cpu().numpy()), dense)
    np.testing.assert_array_equal(
        lists_to_mask(out["q_count"].cpu().numpy(), out["q_idx"].cpu().numpy()), np.swapaxes(dense, 1, 2))
    qa = oracle.pool(q.float().reshape(H, S, D), 64)
    ka = oracle.pool(k.float().reshape(H, S, D), 64)
    p = oracle.reduced_map(qa, ka, 1.0 / np.sqrt(D))
    for h in range(H):
        res = _check_cdf_rows(p[h], dense[h].astype(bool), thr)
        print(f"[chunks] head {h}: kept {int(cnt[0, h].sum())}, CDF rule check {res}", flush=True)
        assert res["unexplained"] == 0, (h, res)
    # The Top-k selector through the same chunks: keep j iff fewer than k entries of
    # its row are strictly larger in the oracle's fp64 map.
    topk = 300
    outk = nb.nabla_build_topk_mask(qg, kg, topk, dense=True)
    torch.cuda.synchronize()
    densek = outk["dense_mask"].cpu().numpy().reshape(H, n, n).astype(bool)
    for h in range(H):
        asc = np.sort(p[h], axis=1)
        above = np.stack([n - np.searchsorted(asc[i], p[h][i], side="right") for i in range(n)])
        np.testing.assert_array_equal(above < topk, densek[h])
    print(f"[chunks] top-{topk}: kept {int(densek.sum())}", flush=True)
    del p
    for h in range(H):
        one = nb.nabla_build_mask(qg[:, h:h + 1].contiguous(), kg[:, h:h + 1].contiguous(), thr)
        onek = nb.nabla_build_topk_mask(qg[:, h:h + 1].contiguous(), kg[:, h:h + 1].contiguous(), topk)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(
            lists_to_mask(one["kv_count"].cpu().numpy(), one["kv_idx"].cpu().numpy())[0], dense[h])
        np.testing.assert_array_equal(
            lists_to_mask(onek["kv_count"].cpu().numpy(), onek["kv_idx"].cpu().numpy())[0].astype(bool), densek[h])


def test_rows_beyond_the_maximum_are_rejected():
    nb = _nb()
    S = 64 * (N_MAX + 1)
    q = torch.zeros((1, 1, S, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nb.NablaError):
        nb.nabla_build_mask(q, q, 0.5)
