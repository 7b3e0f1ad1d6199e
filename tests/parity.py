"""Comparison rules between the HIP path and the CPU oracle.

Mask: the GPU's block mask must equal the oracle's exactly, except
  (a) blocks whose oracle mass-above G_ij lies within BAND (1e-5) of thr -- the
      cumulative-mass band the acceptance rule names; they are counted, and
  (b) blocks whose decision flips under a relative perturbation of REL_TIE of
      the row's probabilities (two probabilities within fp32 rounding of each
      other on opposite sides of the cut: both orders are correct results of
      the same fp32 computation). They are counted too; everything else is an
      unexplained mismatch and fails.
STA-covered blocks are decided by integer logic and are never excused.

Top-k: the same, with the selector's own rule: a mismatch is excused only when
the number of entries that could lie strictly above p_ij under the REL_TIE
perturbation straddles k (p_ij ties with the k-th largest value within fp32
rounding). STA-covered blocks are never excused.

Attention: outputs are compared element by element with the oracle run on the
GPU's own mask, so mask and attention checks stay independent.
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np

BAND = 1e-5
REL_TIE = 1e-4
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3
GRAD_REL_L2 = 1e-2
GRAD_MAX_ABS = 5e-2


def compare_masks(gpu_mask: np.ndarray, orc: Dict[str, np.ndarray], thr: float,
                  sta: Optional[np.ndarray] = None) -> Dict[str, int]:
    gpu = np.asarray(gpu_mask).astype(bool)
    exp = np.asarray(orc["mask"]).astype(bool)
    assert gpu.shape == exp.shape, (gpu.shape, exp.shape)
    g, p = orc["g"], orc["a"]
    mism = gpu != exp
    res = {"blocks": int(exp.size), "kept_oracle": int(exp.sum()), "kept_gpu": int(gpu.sum()),
           "mismatch": int(mism.sum())}
    if thr >= 1.0:
        res.update(band=0, band_mismatch=0, tie_excused=0, unexplained=int(mism.sum()))
        return res
    in_band = np.abs(g - thr) <= BAND
    excusable = np.ones_like(mism) if sta is None else ~np.broadcast_to(sta.astype(bool), mism.shape)
    res["band"] = int((in_band & excusable).sum())
    res["band_mismatch"] = int((mism & in_band & excusable).sum())
    rest = mism & ~in_band & excusable
    tie = 0
    for idx in zip(*np.nonzero(rest)):
        row = p[idx[:-1]]
        pj = row[idx[-1]]
        others = np.delete(row, idx[-1])
        g_lo = others[others > pj * (1 + REL_TIE)].sum()
        g_hi = others[others >= pj * (1 - REL_TIE)].sum()
        if g_lo <= thr + BAND and g_hi >= thr - BAND:
            tie += 1
    res["tie_excused"] = tie
    res["unexplained"] = int((mism & ~(in_band & excusable)).sum()) - tie
    return res


def compare_topk_masks(gpu_mask: np.ndarray, orc: Dict[str, np.ndarray], k: int,
                       sta: Optional[np.ndarray] = None) -> Dict[str, int]:
    gpu = np.asarray(gpu_mask).astype(bool)
    exp = np.asarray(orc["mask"]).astype(bool)
    assert gpu.shape == exp.shape, (gpu.shape, exp.shape)
    p = orc["a"]
    mism = gpu != exp
    excusable = np.ones_like(mism) if sta is None else ~np.broadcast_to(sta.astype(bool), mism.shape)
    tie = 0
    for idx in zip(*np.nonzero(mism & excusable)):
        row = p[idx[:-1]]
        pj = row[idx[-1]]
        others = np.delete(row, idx[-1])
        c_lo = int((others > pj * (1 + REL_TIE)).sum())    # surely above
        c_hi = int((others >= pj * (1 - REL_TIE)).sum())   # possibly above
        if c_lo < k <= c_hi:
            tie += 1
    return {"blocks": int(exp.size), "kept_oracle": int(exp.sum()), "kept_gpu": int(gpu.sum()),
            "mismatch": int(mism.sum()), "tie_excused": tie, "unexplained": int(mism.sum()) - tie}


def lists_to_mask(kv_count: np.ndarray, kv_idx: np.ndarray) -> np.ndarray:
    """Rebuild a dense mask from lists, checking they are strictly ascending and in range."""
    cnt = np.asarray(kv_count)
    idx = np.asarray(kv_idx)
    BH = int(np.prod(cnt.shape[:-1]))
    n = cnt.shape[-1]
    cnt = cnt.reshape(BH, n)
    idx = idx.reshape(BH, n, n)
    m = np.zeros((BH, n, n), dtype=np.uint8)
    assert cnt.min() >= 0 and cnt.max() <= n
    for bh in range(BH):
        for i in range(n):
            js = idx[bh, i, : cnt[bh, i]]
            assert js.size == 0 or (js.min() >= 0 and js.max() < n), (bh, i)
            assert np.all(np.diff(js) > 0), (bh, i)
            m[bh, i, js] = 1
    return m


def attn_errors(gpu: np.ndarray, ref: np.ndarray) -> Dict[str, float]:
    d = np.abs(np.asarray(gpu, dtype=np.float64) - ref)
    return {"max_abs": float(d.max()), "mean_abs": float(d.mean())}


def grad_errors(gpu: np.ndarray, ref: np.ndarray) -> Dict[str, float]:
    g = np.asarray(gpu, dtype=np.float64)
    d = g - ref
    return {"rel_l2": float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30)),
            "max_abs": float(np.abs(d).max())}
