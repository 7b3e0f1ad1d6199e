"""GPU parity of the mask-fidelity diagnostic against the oracle: the dense block
mass (nabla_block_mass) and the per-row recall of block lists against the best
blocks at the same count (nabla_mask_recall)."""

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

# Block mass with the oracle's own LSE: only the bf16-input logits (fp32 MFMA
# sums) and the fp32 exp/sums differ -> relative 1e-4 per entry (plus 1e-7
# absolute for entries that are tiny). With the GPU forward's dense LSE the
# forward's LSE tolerance (1e-3, natural log) enters multiplicatively: rows sum
# to 1 within 2e-3.
MASS_REL = 1e-4
MASS_ABS = 1e-7
ROWSUM_TOL = 2e-3
# Recall: double sums of the same fp32 masses on both sides.
RECALL_TOL = 1e-6


def _nb():
    import block_sparse_attention_nabla_amd as nb
    nb.load_library()
    return nb


def _dense_lse(nb, q, k, v):
    lists = nb.nabla_build_mask(q, k, 1.0)          # thr >= 1 keeps every block
    _, lse = nb.nabla_sparse_attn_fwd(q, k, v, lists["kv_count"], lists["kv_idx"])
    return lse


def _bf16_inputs(name):
    w = synth.get_workload(name)
    x = synth.make_inputs(w)
    return w, {key: x[key].bfloat16() for key in ("q", "k", "v")}


@pytest.mark.parametrize("name,nsamp", [("tiny", None), ("dit_small", 40)])
def test_block_mass_matches_oracle(name, nsamp):
    nb = _nb()
    w, x = _bf16_inputs(name)
    xg = {key: val.cuda() for key, val in x.items()}
    BH, n = w.B * w.H, w.n
    blocks = None
    if nsamp is not None:
        rng = np.random.default_rng(3)
        blocks = sorted(rng.choice(BH * n, nsamp, replace=False).tolist())
    print(f"[fidelity] block mass {name} blocks={'all' if blocks is None else len(blocks)}", flush=True)
    ref = oracle.block_mass(x["q"].float(), x["k"].float(), w.N, blocks=blocks)
    mask_all = np.ones((BH, n, n), dtype=np.uint8)
    _, rlse = oracle.attn_fwd(x["q"].float(), x["k"].float(), x["v"].float(), mask_all, w.N,
                              blocks=blocks)
    rows = ~np.isnan(ref[..., 0])
    # (1) with the oracle's LSE (rows not sampled get a harmless finite value)
    lse_in = torch.from_numpy(np.nan_to_num(rlse, nan=0.0).astype(np.float32)).reshape(w.B, w.H, w.S)
    m1 = nb.nabla_block_mass(xg["q"], xg["k"], lse_in.cuda())
    torch.cuda.synchronize()
    g1 = m1.cpu().numpy().reshape(BH, n, n)
    err = np.abs(g1[rows] - ref[rows])
    bound = MASS_REL * ref[rows] + MASS_ABS
    print(f"[fidelity] oracle-LSE max abs {err.max():.3e}, max rel {(err / np.maximum(ref[rows], 1e-30)).max():.3e}",
          flush=True)
    assert (err <= bound).all()
    # (2) end to end with the GPU's dense LSE
    m2 = nb.nabla_block_mass(xg["q"], xg["k"], _dense_lse(nb, xg["q"], xg["k"], xg["v"]))
    torch.cuda.synchronize()
    sums = m2.sum(dim=-1).cpu().numpy()
    print(f"[fidelity] row sums in [{sums.min():.6f}, {sums.max():.6f}]", flush=True)
    assert np.abs(sums - 1.0).max() <= ROWSUM_TOL


def test_recall_matches_oracle_on_the_same_mass():
    nb = _nb()
    w, x = _bf16_inputs("dit_small")
    xg = {key: val.cuda() for key, val in x.items()}
    mass = nb.nabla_block_mass(xg["q"], xg["k"], _dense_lse(nb, xg["q"], xg["k"], xg["v"]))
    m64 = mass.cpu().numpy().astype(np.float64).reshape(w.B * w.H, w.n, w.n)
    thr = w.thr_for(0.80)
    for label, lists in (
            ("cdf", nb.nabla_build_mask(xg["q"], xg["k"], thr, dense=True)),
            ("topk", nb.nabla_build_topk_mask(xg["q"], xg["k"], 20, dense=True)),
            ("sta", nb.nabla_build_sta_mask(w.B, w.H, w.S, dict(T=w.T, Hs=w.Hs, Ws=w.Ws, P=w.P, win_t=3,
                                                                 win_h=24, win_w=24), "cuda", dense=True))):
        rec, best = nb.nabla_mask_recall(mass, lists["kv_count"], lists["kv_idx"])
        torch.cuda.synchronize()
        mask = lists["dense_mask"].cpu().numpy().reshape(w.B * w.H, w.n, w.n)
        rr, rb = oracle.mask_recall(m64, mask)
        g_rec = rec.cpu().numpy().reshape(rr.shape)
        g_best = best.cpu().numpy().reshape(rb.shape)
        print(f"[fidelity] {label}: mean recall {g_rec.mean():.4f} (best {g_best.mean():.4f}), "
              f"min recall {g_rec.min():.4f}", flush=True)
        np.testing.assert_allclose(g_rec, rr, rtol=RECALL_TOL, atol=RECALL_TOL)
        np.testing.assert_allclose(g_best, rb, rtol=RECALL_TOL, atol=RECALL_TOL)
        assert (g_rec <= g_best + 1e-6).all()


def test_recall_edge_cases():
    nb = _nb()
    B, H, n = 1, 2, 37
    rng = np.random.default_rng(8)
    raw = rng.random((B, H, n, n)).astype(np.float32) ** 4
    raw[0, 0, 3, :] = 0.25                               # a flat row (all tied)
    raw[0, 1, 5, :] = 0.0                                # an all-zero row
    mass = torch.from_numpy(raw).cuda()
    cnt = rng.integers(0, n + 1, (B, H, n)).astype(np.int32)
    cnt[0, 0, 0], cnt[0, 0, 1], cnt[0, 1, 2] = 0, n, 1  # empty, full, single
    idx = np.full((B, H, n, n), -1, dtype=np.int32)
    mask = np.zeros((B * H, n, n), dtype=np.uint8)
    for h in range(H):
        for i in range(n):
            js = np.sort(rng.choice(n, cnt[0, h, i], replace=False))
            idx[0, h, i, :js.size] = js
            mask[h, i, js] = 1
    rec, best = nb.nabla_mask_recall(mass, torch.from_numpy(cnt).cuda(), torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    rr, rb = oracle.mask_recall(raw.astype(np.float64).reshape(B * H, n, n), mask)
    np.testing.assert_allclose(rec.cpu().numpy().reshape(rr.shape), rr, rtol=RECALL_TOL, atol=RECALL_TOL)
    np.testing.assert_allclose(best.cpu().numpy().reshape(rb.shape), rb, rtol=RECALL_TOL, atol=RECALL_TOL)
    assert best[0, 0, 0].item() == 0.0 and rec[0, 0, 0].item() == 0.0


def test_fidelity_720p_sampled():
    # Full 720p layer (40 heads) in the configuration bench.py measures: dense LSE,
    # block mass of every head, recall of the 90% CDF mask; the oracle checks
    # three sampled query blocks' mass rows and their recall.
    nb = _nb()
    w = synth.get_workload("wan14b_720p")
    x = synth.make_inputs(w)
    xg = {key: x[key].cuda() for key in ("q", "k", "v")}
    mass = nb.nabla_block_mass(xg["q"], xg["k"], _dense_lse(nb, xg["q"], xg["k"], xg["v"]))
    lists = nb.nabla_build_mask(xg["q"], xg["k"], w.thr_for(0.90), dense=True)
    rec, best = nb.nabla_mask_recall(mass, lists["kv_count"], lists["kv_idx"])
    torch.cuda.synchronize()
    BH, n = w.B * w.H, w.n
    g = mass.cpu().numpy().reshape(BH, n, n)
    sums = g.sum(axis=-1)
    assert np.abs(sums - 1.0).max() <= ROWSUM_TOL
    blocks = [17, 40 * n // 2 + 611, BH * n - 1]
    ref = oracle.block_mass(x["q"].float(), x["k"].float(), w.N, blocks=blocks)
    for b in blocks:
        bh, i = divmod(b, n)
        r = ref[bh, i]
        # the GPU used its own dense LSE here: entries agree within the row-sum tolerance
        assert np.abs(g[bh, i] - r).max() <= ROWSUM_TOL * r.max() + 1e-6, b
    mask = lists["dense_mask"].cpu().numpy().reshape(BH, n, n)
    rr, rb = oracle.mask_recall(g.astype(np.float64), mask)
    np.testing.assert_allclose(rec.cpu().numpy().reshape(rr.shape), rr, rtol=RECALL_TOL, atol=RECALL_TOL)
    np.testing.assert_allclose(best.cpu().numpy().reshape(rb.shape), rb, rtol=RECALL_TOL, atol=RECALL_TOL)
    print(f"[fidelity] 720p 90%: mean recall {rr.mean():.4f}, best {rb.mean():.4f}, "
          f"min recall {rr.min():.4f}", flush=True)
