"""Comparison rules between the HIP path and the CPU oracle.

Mask (CDF rule, Algorithm 1 of section 3.1.2): the GPU's block mask must equal
the oracle's exactly, except blocks whose oracle mass-above G_ij lies within
BAND (1e-5) of thr -- the cumulative-mass band the acceptance rule names; those
blocks are counted and reported. Every other difference is a failure. (The GPU
resolves the order of nearly equal probabilities next to the cut in fp64, so
fp32 rounding cannot reorder them; see the selection kernel.)

Top-k: the GPU's mask must equal the oracle's exactly (the decision depends on
the order only, which is exact; ties kept together on both sides).

STA-covered blocks are decided by integer logic and are never excused.

Attention: outputs are compared element by element with the oracle run on the
GPU's own mask, so mask and attention checks stay independent.
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np

BAND = 1e-5
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3
GRAD_REL_L2 = 1e-2
GRAD_MAX_ABS = 5e-2
# bf16 keeps 8 significant bits: rounding x to bf16 alone moves it by up to
# 2^-8 |x|, so element-wise gradient checks allow GRAD_MAX_ABS + GRAD_ULP_REL |ref|.
GRAD_ULP_REL = 2.0 ** -8


def compare_masks(gpu_mask: np.ndarray, orc: Dict[str, np.ndarray], thr: float,
                  sta: Optional[np.ndarray] = None) -> Dict[str, int]:
    gpu = np.asarray(gpu_mask).astype(bool)
    exp = np.asarray(orc["mask"]).astype(bool)
    assert gpu.shape == exp.shape, (gpu.shape, exp.shape)
    g = orc["g"]
    mism = gpu != exp
    res = {"blocks": int(exp.size), "kept_oracle": int(exp.sum()), "kept_gpu": int(gpu.sum()),
           "mismatch": int(mism.sum())}
    if thr >= 1.0:
        res.update(band=0, band_mismatch=0, unexplained=int(mism.sum()))
        return res
    in_band = np.abs(g - thr) <= BAND
    excusable = np.ones_like(mism) if sta is None else ~np.broadcast_to(sta.astype(bool), mism.shape)
    res["band"] = int((in_band & excusable).sum())
    res["band_mismatch"] = int((mism & in_band & excusable).sum())
    res["unexplained"] = int((mism & ~(in_band & excusable)).sum())
    if res["unexplained"]:
        # Name the first few offending blocks with their oracle G for the log.
        bad = np.argwhere(mism & ~(in_band & excusable))[:8]
        res["first_unexplained"] = [(tuple(int(v) for v in b), float(g[tuple(b)])) for b in bad]
    return res


def compare_topk_masks(gpu_mask: np.ndarray, orc: Dict[str, np.ndarray], k: int,
                       sta: Optional[np.ndarray] = None) -> Dict[str, int]:
    gpu = np.asarray(gpu_mask).astype(bool)
    exp = np.asarray(orc["mask"]).astype(bool)
    assert gpu.shape == exp.shape, (gpu.shape, exp.shape)
    mism = gpu != exp
    return {"blocks": int(exp.size), "kept_oracle": int(exp.sum()), "kept_gpu": int(gpu.sum()),
            "mismatch": int(mism.sum()), "unexplained": int(mism.sum())}


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
    """rel_l2, max_abs, the largest |ref| and the largest error in units of the
    element-wise bound (GRAD_MAX_ABS + GRAD_ULP_REL |ref|): ``bound_ratio`` <= 1 passes."""
    g = np.asarray(gpu, dtype=np.float64)
    d = g - ref
    ad = np.abs(d)
    return {"rel_l2": float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30)),
            "max_abs": float(ad.max()), "max_ref": float(np.abs(ref).max()),
            "bound_ratio": float((ad / (GRAD_MAX_ABS + GRAD_ULP_REL * np.abs(ref))).max())}


def grad_ok(e: Dict[str, float]) -> bool:
    return e["rel_l2"] <= GRAD_REL_L2 and e["bound_ratio"] <= 1.0
