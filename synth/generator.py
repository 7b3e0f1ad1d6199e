"""Seeded synthetic Q, K, V (and dO) with video-like spatio-temporal locality.

Recipe (per (b, h) pair, one torch generator seeded with ``workload.seed(step)``,
draws made in this order for every head in (b, h) order):

1. F: for each of the D channels an i.i.d. N(0, 1) volume on the latent grid
   T x Hs x Ws, smoothed by a separable Gaussian (sigma = 2 tokens, truncated at
   4 sigma, half-sample-symmetric "reflect" boundary) along all three axes and
   divided by the smoothing's analytic gain so that its variance is ~1.
2. eps_Q, eps_K ~ N(0, noise_std^2).
3. V: either F + eps_V with eps_V ~ N(0, noise_std^2) (``shared_v``) or N(0, 1).
dO (``make_dout``) comes from its own seed stream: N(0, 1).

Q = alpha * (F + eps_Q), K = alpha * (F + eps_K). The shared field gives
neighbouring tokens correlated queries and keys, the locality the NABLA paper's
Appendix D (Figure 9) shows in real video-DiT attention maps.

Tokens are then laid out in block order, the "fractal flattening" of the NABLA
paper's section 3.1.1 (Figure 3): frames outermost (time order kept), then P x P
spatial tiles in row-major order, then the P*P tokens of a tile row-major. Block
i of N = P*P consecutive tokens is one spatial tile of one frame.

Nothing here computes any step of the attention method itself.
"""

from __future__ import annotations

import math
from typing import Dict, Optional

import torch

from .workloads import Workload

SMOOTH_SIGMA = 2.0
SMOOTH_TRUNCATE = 4.0


def gaussian_taps(sigma: float = SMOOTH_SIGMA, truncate: float = SMOOTH_TRUNCATE) -> torch.Tensor:
    """Normalised 1-D Gaussian taps w_k, k = -r..r, r = round(truncate * sigma)."""
    r = int(truncate * sigma + 0.5)
    k = torch.arange(-r, r + 1, dtype=torch.float64)
    w = torch.exp(-0.5 * (k / sigma) ** 2)
    return w / w.sum()


def _reflect_index(L: int, r: int) -> torch.Tensor:
    """Indices of a half-sample-symmetric extension of [0, L) to [-r, L + r)."""
    j = torch.arange(-r, L + r, dtype=torch.int64)
    period = 2 * L
    j = torch.remainder(j, period)
    return torch.where(j >= L, period - 1 - j, j)


def _smooth_axis(x: torch.Tensor, axis: int, taps: torch.Tensor) -> torch.Tensor:
    L = x.shape[axis]
    r = (taps.numel() - 1) // 2
    idx = _reflect_index(L, r).to(x.device)
    xp = x.index_select(axis, idx)
    out = torch.zeros_like(x)
    for k in range(taps.numel()):
        out.add_(xp.narrow(axis, k, L), alpha=float(taps[k]))
    return out


def make_field(D: int, T: int, Hs: int, Ws: int, gen: torch.Generator,
               device: torch.device) -> torch.Tensor:
    """One head's smoothed unit-variance field, shape [D, T, Hs, Ws], fp32."""
    taps = gaussian_taps()
    x = torch.randn((D, T, Hs, Ws), generator=gen, device=device, dtype=torch.float32)
    for axis in (1, 2, 3):
        x = _smooth_axis(x, axis, taps)
    # Variance of a unit-variance white field after the separable 3-D filter.
    gain = float((taps ** 2).sum()) ** 3
    return x.mul_(1.0 / math.sqrt(gain))


def _to_block_order(x: torch.Tensor, P: int) -> torch.Tensor:
    """[D, T, Hs, Ws] -> [S, D] in block order (frame, tile row, tile col, py, px)."""
    D, T, Hs, Ws = x.shape
    tH, tW = Hs // P, Ws // P
    x = x.reshape(D, T, tH, P, tW, P).permute(1, 2, 4, 3, 5, 0)
    return x.reshape(T * Hs * Ws, D)


def block_order_permutation(T: int, Hs: int, Ws: int, P: int) -> torch.Tensor:
    """perm[s] = raster index (t*Hs + y)*Ws + x of the token at block-order position s."""
    raster = torch.arange(T * Hs * Ws, dtype=torch.int64).reshape(1, T, Hs, Ws)
    return _to_block_order(raster, P).reshape(-1)


def round_to_bf16(x: torch.Tensor) -> torch.Tensor:
    """Round to bfloat16 (round-to-nearest-even)."""
    return x.to(torch.bfloat16)


def make_inputs(w: Workload, step: int = 0, device="cpu", alpha: Optional[float] = None,
                heads: Optional[range] = None) -> Dict[str, torch.Tensor]:
    """Q, K, V of shape [B, H, S, D] in block order.

    fp32 workloads return fp32 tensors; bf16 workloads return bf16 tensors
    (round-to-nearest-even). ``alpha`` overrides the calibrated input scale
    (1.0 gives the unscaled inputs the calibration itself measures).
    ``heads`` restricts generation to a range of flattened (b*H + h) heads: the
    draws of earlier heads are still made, so values match a full generation.
    """
    device = torch.device(device)
    if w.Hs % w.P or w.Ws % w.P:
        raise ValueError("latent height and width must be multiples of the tile edge")
    a = w.alpha() if alpha is None else float(alpha)
    out_dtype = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    BH = w.B * w.H
    sel = range(BH) if heads is None else heads
    nsel = len(sel)
    shape = (nsel, w.S, w.D)
    q = torch.empty(shape, dtype=out_dtype, device=device)
    k = torch.empty(shape, dtype=out_dtype, device=device)
    v = torch.empty(shape, dtype=out_dtype, device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed(step))
    grid = (w.D, w.T, w.Hs, w.Ws)
    for bh in range(sel.stop if heads is not None else BH):
        F = make_field(w.D, w.T, w.Hs, w.Ws, gen, device)
        eq = torch.randn(grid, generator=gen, device=device) * w.noise_std
        ek = torch.randn(grid, generator=gen, device=device) * w.noise_std
        if w.shared_v:
            vv = F + torch.randn(grid, generator=gen, device=device) * w.noise_std
        else:
            vv = torch.randn(grid, generator=gen, device=device)
        if bh not in sel:
            continue
        o = bh - sel.start
        q[o] = _to_block_order((F + eq) * a, w.P).to(out_dtype)
        k[o] = _to_block_order((F + ek) * a, w.P).to(out_dtype)
        v[o] = _to_block_order(vv, w.P).to(out_dtype)
    res = {"q": q, "k": k, "v": v}
    if heads is None:
        for key in res:
            res[key] = res[key].reshape(w.B, w.H, w.S, w.D)
    return res


def make_dout(w: Workload, step: int = 0, device="cpu") -> torch.Tensor:
    """dO ~ N(0, 1) of shape [B, H, S, D] (bf16), from its own seed stream."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed(step) + 500)
    x = torch.randn((w.B, w.H, w.S, w.D), generator=gen, device=device)
    return x.to(torch.bfloat16 if w.dtype != "fp32" else torch.float32)
