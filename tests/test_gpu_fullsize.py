"""Parity at the full workload sizes, in the launch configuration the benchmark
times: the GPU runs every head; the oracle checks the mask of every head and
query blocks sampled in every head (attention; backward: sampled query / key
blocks), computed one by one."""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (grad_ok, O_MAX_ABS, O_MEAN_ABS, attn_errors, compare_masks,
                    grad_errors, lists_to_mask)

pytestmark = pytest.mark.gpu


def _nb():
    import block_sparse_attention_nabla_amd as nb
    nb.load_library()
    return nb


_CACHE = {}


def _inputs(name):
    if name not in _CACHE:
        w = synth.get_workload(name)
        print(f"[full] generating {name}", flush=True)
        x = synth.make_inputs(w)
        if w.backward:
            x["do"] = synth.make_dout(w)
        _CACHE.clear()
        _CACHE[name] = (w, x, {k: v.cuda() for k, v in x.items()})
    return _CACHE[name]


def _mask_sampled(w, x, out, thr, heads):
    n = w.n
    dense = out["dense_mask"].reshape(w.B * w.H, n, n)
    res_all = []
    for bh in heads:
        orc = oracle.build_mask(x["q"].reshape(-1, w.S, w.D)[bh:bh + 1].float(),
                                x["k"].reshape(-1, w.S, w.D)[bh:bh + 1].float(), w.N, thr,
                                sta=w.sta_struct())
        res = compare_masks(dense[bh:bh + 1].cpu().numpy(), orc, thr)
        res_all.append(res)
        assert res["unexplained"] == 0, (bh, res)
    tot = {key: sum(r[key] for r in res_all) for key in res_all[0]}
    print(f"[full] mask {w.name} thr={thr:.4f} heads={len(res_all)} totals {tot}", flush=True)


def _fwd_sampled(w, x, xg, lists, mask, per_head, seed):
    # The benchmark's configuration: the frame hint (paired query blocks); the
    # unpaired kernel must give the same bits.
    nb = _nb()
    fb = (w.Hs // w.P) * (w.Ws // w.P)
    o, lse = nb.nabla_sparse_attn_fwd(xg["q"], xg["k"], xg["v"], lists["kv_count"], lists["kv_idx"],
                                      frame_blocks=fb)
    o0, lse0 = nb.nabla_sparse_attn_fwd(xg["q"], xg["k"], xg["v"], lists["kv_count"], lists["kv_idx"])
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o0.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse0.view(torch.int32))
    del o0, lse0
    rng = np.random.default_rng(seed)
    blocks = sorted(bh * w.n + int(i) for bh in range(w.B * w.H)
                    for i in rng.choice(w.n, per_head, replace=False))
    # Always include the longest and the shortest list.
    cnt = lists["kv_count"].reshape(-1).cpu().numpy()
    blocks = sorted(set(blocks) | {int(cnt.argmax()), int(cnt.argmin())})
    ro, rlse = oracle.attn_fwd(x["q"].float(), x["k"].float(), x["v"].float(), mask, w.N, blocks=blocks)
    of = o.float().cpu().numpy().reshape(w.B * w.H, w.S, w.D)
    sel = ~np.isnan(ro[..., 0])
    e = attn_errors(of[sel], ro[sel])
    dl = float(np.abs(lse.cpu().numpy().reshape(w.B * w.H, w.S)[sel] - rlse[sel]).max())
    print(f"[full] fwd {w.name} sampled blocks={len(blocks)} {e} lse_max_abs={dl:.2e}", flush=True)
    assert e["max_abs"] <= O_MAX_ABS and e["mean_abs"] <= O_MEAN_ABS, e
    assert dl <= 1e-3
    return o, lse


@pytest.mark.parametrize("sparsity", [0.80, 0.90])
def test_wan14b_720p_mask_and_forward(sparsity):
    nb = _nb()
    w, x, xg = _inputs("wan14b_720p")
    thr = w.thr_for(sparsity)
    print(f"[full] wan14b_720p sparsity={sparsity} thr={thr}", flush=True)
    out = nb.nabla_build_mask(xg["q"], xg["k"], thr, dense=True)
    torch.cuda.synchronize()
    kept = int(out["kv_count"].sum())
    achieved = 1.0 - kept / (w.B * w.H * w.n * w.n)
    print(f"[full] achieved sparsity {achieved:.5f}", flush=True)
    assert abs(achieved - sparsity) < 0.005
    _mask_sampled(w, x, out, thr, heads=range(w.B * w.H))
    mask = out["dense_mask"].reshape(w.B * w.H, w.n, w.n).cpu().numpy()
    _fwd_sampled(w, x, xg, out, mask, per_head=6, seed=int(sparsity * 100))


def test_dit2b_train_mask_forward_backward():
    nb = _nb()
    w, x, xg = _inputs("dit2b_train")
    thr = w.thr_for(0.85)
    out = nb.nabla_build_mask(xg["q"], xg["k"], thr, transpose=True, dense=True)
    torch.cuda.synchronize()
    _mask_sampled(w, x, out, thr, heads=range(w.B * w.H))
    mask = out["dense_mask"].reshape(w.B * w.H, w.n, w.n).cpu().numpy()
    o, lse = _fwd_sampled(w, x, xg, out, mask, per_head=6, seed=5)
    np.testing.assert_array_equal(lists_to_mask(out["q_count"].cpu().numpy(), out["q_idx"].cpu().numpy()),
                                  np.swapaxes(mask, 1, 2))
    dq, dk, dv = nb.nabla_sparse_attn_bwd(xg["q"], xg["k"], xg["v"], o, xg["do"], lse, out["kv_count"],
                                          out["kv_idx"], out["q_count"], out["q_idx"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    # Two query blocks (dQ) and two key blocks (dK, dV) sampled in every head, plus
    # each head's longest loops: the query block with the most kept key blocks
    # (dQ) and the key block kept by the most query blocks (dK, dV).
    kvc = out["kv_count"].reshape(w.B * w.H, w.n).cpu().numpy()
    qc = out["q_count"].reshape(w.B * w.H, w.n).cpu().numpy()
    qb = sorted({bh * w.n + int(i) for bh in range(w.B * w.H) for i in rng.choice(w.n, 2, replace=False)}
                | {bh * w.n + int(kvc[bh].argmax()) for bh in range(w.B * w.H)})
    kb = sorted({bh * w.n + int(i) for bh in range(w.B * w.H) for i in rng.choice(w.n, 2, replace=False)}
                | {bh * w.n + int(qc[bh].argmax()) for bh in range(w.B * w.H)})
    print(f"[full] bwd longest loops: dQ up to {kvc.max()} key blocks, dK/dV up to {qc.max()} query blocks",
          flush=True)
    rdq, rdk, rdv = oracle.attn_bwd(x["q"].float(), x["k"].float(), x["v"].float(), x["do"].float(), mask,
                                    w.N, q_blocks=qb, kv_blocks=kb)
    res = {}
    for name, g, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        gg = g.float().cpu().numpy().reshape(w.B * w.H, w.S, w.D)
        sel = ~np.isnan(r[..., 0])
        res[name] = grad_errors(gg[sel], r[sel])
        assert grad_ok(res[name]), (name, res)
    print(f"[full] bwd dit2b_train {res}", flush=True)
