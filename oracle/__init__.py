"""CPU oracle for the NABLA hot path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package. It is a plain, slow, fp64-accumulating reference
written from "NABLA: Neighborhood Adaptive Block-Level Attention" (arXiv
2507.13546): eq. (2)-(5) and Algorithm 1. It shares no code with the HIP
library. The heavy loops live in ``nabla_oracle.c`` (plain C + OpenMP); this
module only marshals numpy arrays.

Every function here is pinned by ``tests/test_oracle_*.py`` against facts fixed
independently of this code (library routines, brute force, closed forms and the
paper's Table 1).
"""

from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nabla_oracle.c")
_LIB = os.path.join(_HERE, "libnabla_oracle.so")
_lib = None

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_dbl = ctypes.c_double
_vp = ctypes.c_void_p


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, IEEE arithmetic: no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                        "-fvisibility=hidden", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = ctypes.CDLL(_LIB)
    lib.nabla_oracle_num_threads.restype = ctypes.c_int
    lib.nabla_oracle_pool.argtypes = [_f32p, _i64, _i64, _i64, _i64, _f64p]
    lib.nabla_oracle_reduced_map.argtypes = [_f64p, _f64p, _i64, _i64, _i64, _dbl, _f64p]
    lib.nabla_oracle_mass_above.argtypes = [_f64p, _i64, _i64, _f64p]
    lib.nabla_oracle_cdf_mask.argtypes = [_f64p, _i64, _dbl, _u8p]
    lib.nabla_oracle_count_above.argtypes = [_f64p, _i64, _i64, _i64p]
    lib.nabla_oracle_block_mass.argtypes = [_f32p, _f32p, _i64, _i64, _i64, _i64, _dbl, _vp, _i64,
                                            _f64p]
    lib.nabla_oracle_sta_mask.argtypes = [_i64] * 7 + [_u8p]
    lib.nabla_oracle_union.argtypes = [_u8p, _u8p, _i64, _i64]
    lib.nabla_oracle_attn_fwd.argtypes = [_f32p, _f32p, _f32p, _i64, _i64, _i64, _i64, _u8p,
                                          _dbl, _vp, _i64, _f64p, _f64p]
    lib.nabla_oracle_attn_bwd_dq.argtypes = [_f32p, _f32p, _f32p, _f32p, _i64, _i64, _i64, _i64,
                                             _u8p, _dbl, _vp, _i64, _f64p]
    lib.nabla_oracle_attn_bwd_dkdv.argtypes = [_f32p, _f32p, _f32p, _f32p, _i64, _i64, _i64,
                                               _i64, _u8p, _dbl, _vp, _i64, _f64p, _f64p]
    _lib = lib
    return lib


def num_threads() -> int:
    return int(_load().nabla_oracle_num_threads())


def _as_f32(x) -> np.ndarray:
    """Accept numpy or torch (any float dtype); return C-contiguous fp32 [BH, S, D]."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").float().numpy()
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 4:
        x = x.reshape(-1, x.shape[-2], x.shape[-1])
    if x.ndim != 3:
        raise ValueError("expected [B, H, S, D] or [BH, S, D]")
    return x


def pool(x, N: int) -> np.ndarray:
    """Algorithm 1, steps 2-5: block means over N tokens -> [BH, S/N, D] (fp64)."""
    x = _as_f32(x)
    BH, S, D = x.shape
    if S % N:
        raise ValueError("S must be a multiple of N")
    out = np.empty((BH, S // N, D), dtype=np.float64)
    _load().nabla_oracle_pool(x, BH, S, D, N, out)
    return out


def reduced_map(qa: np.ndarray, ka: np.ndarray, scale: float) -> np.ndarray:
    """Algorithm 1, steps 6-7: row softmax of Q_a K_a^T * scale -> [BH, n, n] (fp64)."""
    qa = np.ascontiguousarray(qa, dtype=np.float64)
    ka = np.ascontiguousarray(ka, dtype=np.float64)
    BH, n, D = qa.shape
    a = np.empty((BH, n, n), dtype=np.float64)
    _load().nabla_oracle_reduced_map(qa, ka, BH, n, D, float(scale), a)
    return a


def mass_above(a: np.ndarray) -> np.ndarray:
    """G_ij = sum of row i's entries strictly larger than entry j -> [BH, n, n]."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    BH, n, _ = a.shape
    g = np.empty_like(a)
    _load().nabla_oracle_mass_above(a, BH, n, g)
    return g


def cdf_mask(g: np.ndarray, thr: float) -> np.ndarray:
    """Algorithm 1, step 10 in G form: keep iff thr >= 1 or G <= thr (uint8)."""
    if not (thr >= 0.0) or math.isnan(thr):
        raise ValueError("thr must be a finite number >= 0")
    g = np.ascontiguousarray(g, dtype=np.float64)
    m = np.empty(g.shape, dtype=np.uint8)
    _load().nabla_oracle_cdf_mask(g, g.size, float(thr), m)
    return m


def count_above(a: np.ndarray) -> np.ndarray:
    """C_ij = number of entries of row i strictly larger than entry j -> [BH, n, n] int64."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    BH, n, _ = a.shape
    c = np.empty(a.shape, dtype=np.int64)
    _load().nabla_oracle_count_above(a, BH, n, c)
    return c


def topk_mask(a: np.ndarray, k: int) -> np.ndarray:
    """Top-k selector: keep j iff fewer than k entries of its row are strictly larger (uint8).

    Keeps the k largest entries of every row; entries tied at the k-th value are
    kept together. k must be >= 1."""
    if int(k) < 1:
        raise ValueError("k must be >= 1")
    return (count_above(a) < int(k)).astype(np.uint8)


def sta_only_mask(BH: int, T: int, Hs: int, Ws: int, P: int, win_t: int, win_h: int,
                  win_w: int) -> np.ndarray:
    """The static STA selector on its own: the STA map for every head -> [BH, n, n] uint8."""
    m = sta_mask(T, Hs, Ws, P, win_t, win_h, win_w)
    return np.ascontiguousarray(np.broadcast_to(m, (BH,) + m.shape))


def sta_mask(T: int, Hs: int, Ws: int, P: int, win_t: int, win_h: int, win_w: int) -> np.ndarray:
    """STA block map [n, n]: clipped window centred on the query tile (section 2.2, eq. (4))."""
    n = T * (Hs // P) * (Ws // P)
    m = np.empty((n, n), dtype=np.uint8)
    _load().nabla_oracle_sta_mask(T, Hs, Ws, P, win_t, win_h, win_w, m)
    return m


def union(mask: np.ndarray, sta: np.ndarray) -> np.ndarray:
    """Section 3.1.3: M = M_nabla OR M_STA (returns a new array)."""
    m = np.ascontiguousarray(mask, dtype=np.uint8).copy()
    BH, n, _ = m.shape
    _load().nabla_oracle_union(m, np.ascontiguousarray(sta, dtype=np.uint8), BH, n)
    return m


def build_mask(q, k, N: int, thr: float, sta: Optional[Dict[str, int]] = None,
               scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """The whole mask stage: pool, reduced softmax, CDF binarisation, optional STA union.

    Returns the final block mask plus the intermediate fp64 map ``a`` and masses ``g``.
    """
    qa, ka = pool(q, N), pool(k, N)
    D = qa.shape[-1]
    a = reduced_map(qa, ka, (1.0 / math.sqrt(D)) if scale is None else scale)
    g = mass_above(a)
    m = cdf_mask(g, thr)
    nab = m
    if sta is not None:
        s = sta_mask(sta["T"], sta["Hs"], sta["Ws"], sta["P"], sta["win_t"], sta["win_h"],
                     sta["win_w"])
        m = union(m, s)
    return {"mask": m, "mask_nabla": nab, "a": a, "g": g, "qa": qa, "ka": ka}


def build_topk_mask(q, k, N: int, topk: int, sta: Optional[Dict[str, int]] = None,
                    scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Mask stage with the Top-k selector in place of the CDF rule: pool, reduced
    softmax, keep the top-k blocks of every row, optional STA union."""
    qa, ka = pool(q, N), pool(k, N)
    D = qa.shape[-1]
    a = reduced_map(qa, ka, (1.0 / math.sqrt(D)) if scale is None else scale)
    m = topk_mask(a, topk)
    sel = m
    if sta is not None:
        s = sta_mask(sta["T"], sta["Hs"], sta["Ws"], sta["P"], sta["win_t"], sta["win_h"],
                     sta["win_w"])
        m = union(m, s)
    return {"mask": m, "mask_topk": sel, "a": a, "qa": qa, "ka": ka}


def mask_to_lists(mask: np.ndarray) -> Dict[str, np.ndarray]:
    """Compact a block mask [BH, n, n] to per-row ascending index lists and the transpose.

    kv_count[bh, i] = #kept j; kv_idx[bh, i, :kv_count] = kept j ascending (rest -1).
    q_count[bh, j] = #i keeping j; q_idx[bh, j, :q_count] = those i ascending (rest -1).
    """
    m = np.asarray(mask).astype(bool)
    BH, n, _ = m.shape
    kv_count = m.sum(axis=2).astype(np.int32)
    q_count = m.sum(axis=1).astype(np.int32)
    kv_idx = np.full((BH, n, n), -1, dtype=np.int32)
    q_idx = np.full((BH, n, n), -1, dtype=np.int32)
    for bh in range(BH):
        for i in range(n):
            js = np.nonzero(m[bh, i])[0]
            kv_idx[bh, i, : js.size] = js
        for j in range(n):
            is_ = np.nonzero(m[bh, :, j])[0]
            q_idx[bh, j, : is_.size] = is_
    return {"kv_count": kv_count, "kv_idx": kv_idx, "q_count": q_count, "q_idx": q_idx}


def _blocks_arg(blocks: Optional[Sequence[int]]) -> Tuple[Optional[np.ndarray], int]:
    if blocks is None:
        return None, 0
    arr = np.ascontiguousarray(np.asarray(blocks, dtype=np.int64))
    return arr, int(arr.size)


def attn_fwd(q, k, v, mask: np.ndarray, N: int, scale: Optional[float] = None,
             blocks: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Masked attention, eq. (4), on kept blocks. Returns O [BH, S, D] and LSE [BH, S] (fp64).

    ``blocks`` restricts the computation to flattened query blocks (bh*n + i);
    other rows are left as NaN.
    """
    q, k, v = _as_f32(q), _as_f32(k), _as_f32(v)
    BH, S, D = q.shape
    m = np.ascontiguousarray(mask, dtype=np.uint8).reshape(BH, S // N, S // N)
    sc = (1.0 / math.sqrt(D)) if scale is None else float(scale)
    o = np.full((BH, S, D), np.nan, dtype=np.float64)
    lse = np.full((BH, S), np.nan, dtype=np.float64)
    arr, cnt = _blocks_arg(blocks)
    ptr = arr.ctypes.data if arr is not None else None
    _load().nabla_oracle_attn_fwd(q, k, v, BH, S, D, N, m, sc, ptr, cnt, o, lse)
    return o, lse


def attn_bwd(q, k, v, dout, mask: np.ndarray, N: int, scale: Optional[float] = None,
             q_blocks: Optional[Sequence[int]] = None,
             kv_blocks: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of eq. (4) with the mask held constant: dQ, dK, dV [BH, S, D] (fp64).

    ``q_blocks`` / ``kv_blocks`` restrict dQ rows / dK, dV rows to the listed
    flattened blocks; other rows are NaN.
    """
    q, k, v, dout = _as_f32(q), _as_f32(k), _as_f32(v), _as_f32(dout)
    BH, S, D = q.shape
    m = np.ascontiguousarray(mask, dtype=np.uint8).reshape(BH, S // N, S // N)
    sc = (1.0 / math.sqrt(D)) if scale is None else float(scale)
    dq = np.full((BH, S, D), np.nan, dtype=np.float64)
    dk = np.full((BH, S, D), np.nan, dtype=np.float64)
    dv = np.full((BH, S, D), np.nan, dtype=np.float64)
    lib = _load()
    arr, cnt = _blocks_arg(q_blocks)
    lib.nabla_oracle_attn_bwd_dq(q, k, v, dout, BH, S, D, N, m, sc,
                                 arr.ctypes.data if arr is not None else None, cnt, dq)
    arr2, cnt2 = _blocks_arg(kv_blocks)
    lib.nabla_oracle_attn_bwd_dkdv(q, k, v, dout, BH, S, D, N, m, sc,
                                   arr2.ctypes.data if arr2 is not None else None, cnt2, dk, dv)
    return dq, dk, dv


# ----------------------------------------------------------------------------
# Token reordering, section 3.1.1 (Figure 3): "fractal flattening". Each P x P
# spatial patch of a frame becomes P*P consecutive tokens; frames keep their
# time order. Raster order is (t, y, x) with x fastest.
# ----------------------------------------------------------------------------
def token_order(T: int, Hs: int, Ws: int, P: int) -> np.ndarray:
    """perm[s] = raster index of the token at block-order position s."""
    if Hs % P or Ws % P:
        raise ValueError("frame height and width must be multiples of P")
    tH, tW = Hs // P, Ws // P
    perm = np.empty(T * Hs * Ws, dtype=np.int64)
    s = 0
    for t in range(T):
        for ty in range(tH):
            for tx in range(tW):
                for py in range(P):
                    for px in range(P):
                        y, x = ty * P + py, tx * P + px
                        perm[s] = (t * Hs + y) * Ws + x
                        s += 1
    return perm


def tokens_to_blocks(x: np.ndarray, T: int, Hs: int, Ws: int, P: int) -> np.ndarray:
    """Rows of x (axis -2: tokens in raster order) into block order."""
    return np.ascontiguousarray(x[..., token_order(T, Hs, Ws, P), :])


def blocks_to_tokens(x: np.ndarray, T: int, Hs: int, Ws: int, P: int) -> np.ndarray:
    """Inverse of tokens_to_blocks: rows in block order back to raster order."""
    out = np.empty_like(x)
    out[..., token_order(T, Hs, Ws, P), :] = x
    return out


# ----------------------------------------------------------------------------
# Mask-fidelity diagnostic: the per-block fidelity test the review record of
# arXiv 2507.13546 (pith.science) asks for -- how much of full attention's
# token-level probability mass falls inside the kept blocks, against the best
# blocks one could keep with the same per-row budget.
# ----------------------------------------------------------------------------
def block_mass(q, k, N: int, scale: Optional[float] = None,
               blocks: Optional[Sequence[int]] = None) -> np.ndarray:
    """M_ij = mean over the N queries of block i of the dense softmax mass on key block j.

    Returns [BH, n, n] fp64; rows not listed in ``blocks`` are NaN."""
    q, k = _as_f32(q), _as_f32(k)
    BH, S, D = q.shape
    n = S // N
    sc = (1.0 / math.sqrt(D)) if scale is None else float(scale)
    m = np.full((BH, n, n), np.nan, dtype=np.float64)
    arr, cnt = _blocks_arg(blocks)
    _load().nabla_oracle_block_mass(q, k, BH, S, D, N, sc,
                                    arr.ctypes.data if arr is not None else None, cnt, m)
    return m


def mask_recall(mass: np.ndarray, mask: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per row: (mass inside the kept blocks, mass inside the c best blocks), c = kept count.

    The second is the top-mass block oracle at the same per-row budget: the sum of
    the row's c largest block masses (a sort; ties do not change the sum)."""
    mass = np.asarray(mass, dtype=np.float64)
    keep = np.asarray(mask).astype(bool)
    recall = np.where(keep, mass, 0.0).sum(axis=-1)
    c = keep.sum(axis=-1)
    desc = -np.sort(-mass, axis=-1)
    csum = np.concatenate([np.zeros(mass.shape[:-1] + (1,)), np.cumsum(desc, axis=-1)], axis=-1)
    best = np.take_along_axis(csum, c[..., None], axis=-1)[..., 0]
    return recall, best
