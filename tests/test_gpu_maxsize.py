"""The largest supported row: n = 8192 blocks per head (S = 524,288 tokens).

At this size the oracle's selection (quadratic per row) would take minutes, so the
GPU mask is checked against the definition of the CDF rule on the oracle's fp64
reduced map, row by row (section 3.1.2): the kept set is an upper set of the row
(every entry larger than a kept one is kept), its mass exceeds thr, and dropping
its smallest tie group brings the mass to thr or below -- up to the same 1e-5
band and fp32 ties the other parity tests allow. Forward (with and without the
frame hint, bitwise equal) and backward are checked on sampled blocks against the
oracle run on the GPU's own mask."""

import numpy as np
import pytest
import torch

import oracle
from parity import (BAND, GRAD_MAX_ABS, GRAD_REL_L2, LSE_MAX_ABS, O_MAX_ABS, O_MEAN_ABS, REL_TIE,
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
    bad = 0
    for i in range(p.shape[0]):
        row, kr = p[i], keep[i]
        kept_vals = row[kr]
        assert kept_vals.size >= 1, i
        lo = kept_vals.min()
        # upper set: nothing clearly above the smallest kept value is dropped
        dropped_above = (~kr) & (row > lo * (1 + REL_TIE))
        # mass of the kept set exceeds thr (G of the smallest kept entry <= thr)
        g_lo = row[row > lo * (1 + REL_TIE)].sum()
        # minimality: G of the largest dropped entry > thr
        if (~kr).any():
            hi_dropped = row[~kr].max()
            g_hi = row[row > hi_dropped * (1 + REL_TIE)].sum()
            minimal = g_hi > thr - BAND or hi_dropped >= lo * (1 - REL_TIE)
        else:
            minimal = True
        if dropped_above.any() or g_lo > thr + BAND or not minimal:
            bad += 1
    return {"rows": int(p.shape[0]), "bad_rows": bad}


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
    assert res["bad_rows"] == 0, res
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
    qb = [5, N_MAX - 2]
    qc = out["q_count"][0, 0].cpu().numpy()
    kb = [int(np.argmin(np.where(qc > 0, qc, N_MAX + 1))), 9]  # the oracle's cost grows with q_count
    rdq, rdk, rdv = oracle.attn_bwd(q.float(), k.float(), v.float(), do.float(), dense, 64,
                                    q_blocks=qb, kv_blocks=kb)
    res = {}
    for name, g_, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        gg = g_.float().cpu().numpy().reshape(1, S, D)
        m = ~np.isnan(r[..., 0])
        res[name] = grad_errors(gg[m], r[m])
        assert res[name]["rel_l2"] <= GRAD_REL_L2 and res[name]["max_abs"] <= GRAD_MAX_ABS, (name, res)
    print(f"[max] bwd sampled {res}", flush=True)


def test_rows_beyond_the_maximum_are_rejected():
    nb = _nb()
    S = 64 * (N_MAX + 1)
    q = torch.zeros((1, 1, S, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nb.NablaError):
        nb.nabla_build_mask(q, q, 0.5)
