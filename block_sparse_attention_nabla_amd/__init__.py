"""NABLA block-sparse attention for MI355X (gfx950): Python binding of libnabla.

Argument marshalling only: every step of the path runs in the HIP kernels of
``libnabla.so``, called through its C ABI (``include/nabla.h``). PyTorch is used
for device memory and the current HIP stream. There is no CPU fallback: if the
library is not built, every call raises.

Entry points (same names as the C ABI):
    nabla_build_mask(q, k, thr, sta=None, ...)      -> dict of block lists
    nabla_build_topk_mask(q, k, topk, sta=None, ...) -> dict of block lists (Top-k selector)
    nabla_build_sta_mask(B, H, S, sta, device, ...)  -> dict of block lists (STA alone)
    nabla_sparse_attn_fwd(q, k, v, kv_count, kv_idx) -> (o, lse)
    nabla_sparse_attn_bwd(q, k, v, o, d_o, lse, kv_count, kv_idx, q_count, q_idx)
                                                     -> (dq, dk, dv)
    nabla_reorder_tokens(x, T, Hs, Ws, P, inverse=False) -> reordered copy
    nabla_block_mass(q, k, lse)                      -> dense block masses [B,H,n,n]
    nabla_mask_recall(mass, kv_count, kv_idx)        -> (recall, best_recall) per row
    nabla_check_lists(count, idx)                    -> number of malformed list rows
    nabla_workspace_size(op, B, H, S, D, N), nabla_status_string(code)

Streams: every entry point launches on ``stream`` (a torch.cuda.Stream), else on
the current stream. With an explicit stream, the tensors a call allocates
(outputs, workspace) are allocated on that stream too, so the caching allocator
never hands them to other work while the call's kernels may still use them.
"""

from __future__ import annotations

import ctypes
import functools
import math
import os
from typing import Dict, Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnabla.so")

NABLA_OK = 0
NABLA_OP_MASK, NABLA_OP_FWD, NABLA_OP_BWD, NABLA_OP_STA_MASK = 0, 1, 2, 3
NABLA_DTYPE_BF16, NABLA_DTYPE_FP32 = 0, 1
BLOCK_N = 64

EXPORTED_SYMBOLS = (
    "nabla_workspace_size",
    "nabla_status_string",
    "nabla_build_mask",
    "nabla_build_topk_mask",
    "nabla_build_sta_mask",
    "nabla_sparse_attn_fwd",
    "nabla_sparse_attn_fwd_static",
    "nabla_sparse_attn_bwd",
    "nabla_reorder_tokens",
    "nabla_block_mass",
    "nabla_mask_recall",
    "nabla_check_lists",
)


class NablaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {nabla_status_string(status)} ({status})")


class StaWindow(ctypes.Structure):
    """nabla_sta_t: latent grid T x Hs x Ws, tile edge P, window in tokens."""
    _fields_ = [(name, ctypes.c_int32) for name in ("T", "Hs", "Ws", "P", "win_t", "win_h", "win_w")]


_lib = None
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libnabla.so (built by ``python -m block_sparse_attention_nabla_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m block_sparse_attention_nabla_amd.build`")
    lib = ctypes.CDLL(path)
    lib.nabla_workspace_size.restype = ctypes.c_size_t
    lib.nabla_workspace_size.argtypes = [_i32] * 6
    lib.nabla_status_string.restype = ctypes.c_char_p
    lib.nabla_status_string.argtypes = [ctypes.c_int]
    lib.nabla_build_mask.restype = ctypes.c_int
    lib.nabla_build_mask.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _i32, ctypes.c_float,
                                     ctypes.POINTER(StaWindow), _vp, _vp, _vp, _vp, _vp, _vp,
                                     ctypes.c_size_t, _vp]
    lib.nabla_build_topk_mask.restype = ctypes.c_int
    lib.nabla_build_topk_mask.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                          ctypes.POINTER(StaWindow), _vp, _vp, _vp, _vp, _vp, _vp,
                                          ctypes.c_size_t, _vp]
    lib.nabla_build_sta_mask.restype = ctypes.c_int
    lib.nabla_build_sta_mask.argtypes = [_i32, _i32, _i32, _i32, ctypes.POINTER(StaWindow), _vp, _vp,
                                         _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.nabla_sparse_attn_fwd.restype = ctypes.c_int
    lib.nabla_sparse_attn_fwd.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                          ctypes.c_float, _i32, _vp, _i32, _vp, _vp, ctypes.c_size_t,
                                          _vp]
    lib.nabla_sparse_attn_fwd_static.restype = ctypes.c_int
    lib.nabla_sparse_attn_fwd_static.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                                 ctypes.c_float, _i32, _vp, _i32, _vp, _vp]
    lib.nabla_sparse_attn_bwd.restype = ctypes.c_int
    lib.nabla_sparse_attn_bwd.argtypes = [_vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                                          _i32, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp,
                                          _vp, ctypes.c_size_t, _vp]
    lib.nabla_block_mass.restype = ctypes.c_int
    lib.nabla_block_mass.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _vp,
                                     _vp]
    lib.nabla_mask_recall.restype = ctypes.c_int
    lib.nabla_mask_recall.argtypes = [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp]
    lib.nabla_check_lists.restype = ctypes.c_int
    lib.nabla_check_lists.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp]
    lib.nabla_reorder_tokens.restype = ctypes.c_int
    lib.nabla_reorder_tokens.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _i32, ctypes.c_int64,
                                         _i32, _vp]
    _lib = lib
    return lib


def nabla_status_string(status: int) -> str:
    return load_library().nabla_status_string(int(status)).decode()


def nabla_workspace_size(op: int, B: int, H: int, S: int, D: int, N: int = BLOCK_N) -> int:
    return int(load_library().nabla_workspace_size(op, B, H, S, D, N))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor, stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _on_stream(fn):
    """Run an entry point with ``stream`` (when given) as the current stream, so
    that its allocations belong to the stream its kernels run on."""

    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kwargs):
        if stream is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kwargs)

    return wrapper


def _check_qkv(name: str, t: torch.Tensor, shape=None):
    """Shape/dtype/layout of a [B, H, S, D] bf16 input (the device is checked by _check_devices)."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_contiguous() \
            or t.dim() != 4:
        raise ValueError(f"{name} must be a contiguous bfloat16 tensor [B, H, S, D]")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_tensor(name: str, t, dtypes, shape):
    """dtype (one of ``dtypes``), exact shape and contiguity of a tensor argument."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    dts = dtypes if isinstance(dtypes, tuple) else (dtypes,)
    if t.dtype not in dts:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {' or '.join(str(d) for d in dts)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_devices(device: torch.device, **tensors):
    """Every tensor handed to the library must live on ``device``, a CUDA (HIP) device."""
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a CUDA (HIP) device, got {device}")
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _workspace(op, B, H, S, D, N, device, workspace):
    size = nabla_workspace_size(op, B, H, S, D, N)
    if workspace is None:
        if device.type != "cuda":
            raise ValueError(f"tensors must be on a CUDA (HIP) device, got {device}")
        workspace = torch.empty(max(size, 1), dtype=torch.uint8, device=device)
    else:
        _check_tensor("workspace", workspace, torch.uint8, None)
        if workspace.numel() < size:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, needs {size}")
        _check_devices(device, workspace=workspace)
    return workspace, size


def _mask_outputs(B, H, n, dev, transpose, dense, out, allocate=True):
    """Check caller-provided mask outputs (shape and dtype first, then device) and
    allocate the missing ones on ``dev``; with allocate=False, only the shape and
    dtype checks."""
    out = dict(out or {})
    keys = [("kv_count", (B, H, n), torch.int32), ("kv_idx", (B, H, n, n), torch.int32)]
    if transpose:
        keys += [("q_count", (B, H, n), torch.int32), ("q_idx", (B, H, n, n), torch.int32)]
    if dense:
        keys += [("dense_mask", (B, H, n, n), torch.uint8)]
    given = {}
    for key, shape, dtype in keys:
        t = out.get(key)
        if t is not None:
            _check_tensor(f"out[{key!r}]", t, dtype, shape)
            given[f"out[{key!r}]"] = t
    if not allocate:
        return None
    _check_devices(dev, **given)
    return {key: out[key] if out.get(key) is not None else torch.empty(shape, dtype=dtype, device=dev)
            for key, shape, dtype in keys}


def _sta_ptr(sta: Optional[dict]):
    if sta is None:
        return None
    return ctypes.pointer(StaWindow(*(int(sta[f]) for f in ("T", "Hs", "Ws", "P", "win_t", "win_h", "win_w"))))


def _content_mask(fn_name, q, k, select_arg, sta, N, transpose, dense, out, workspace, stream):
    _check_qkv("q", q)
    B, H, S, D = q.shape
    _check_qkv("k", k, q.shape)
    _mask_outputs(B, H, S // N, q.device, transpose, dense, out, allocate=False)
    ws, size = _workspace(NABLA_OP_MASK, B, H, S, D, N, q.device, workspace)
    _check_devices(q.device, k=k)
    res = _mask_outputs(B, H, S // N, q.device, transpose, dense, out)
    st = getattr(load_library(), fn_name)(
        _ptr(q), _ptr(k), B, H, S, D, N, select_arg, _sta_ptr(sta), _ptr(res["kv_count"]),
        _ptr(res["kv_idx"]), _ptr(res.get("q_count")), _ptr(res.get("q_idx")),
        _ptr(res.get("dense_mask")), _ptr(ws), ws.numel(), _stream(q, stream))
    if st != NABLA_OK:
        raise NablaError(st, fn_name)
    return res


@_on_stream
def nabla_build_mask(q: torch.Tensor, k: torch.Tensor, thr: float, sta: Optional[dict] = None,
                     N: int = BLOCK_N, *, transpose: bool = False, dense: bool = False,
                     out: Optional[Dict[str, torch.Tensor]] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> Dict[str, torch.Tensor]:
    """Block mask of section 3.1.2 (Algorithm 1) [+ STA union of section 3.1.3] as lists.

    Returns kv_count [B,H,n], kv_idx [B,H,n,n] and, if requested, q_count / q_idx
    (``transpose``) and dense_mask uint8 [B,H,n,n] (``dense``). ``sta`` holds
    T, Hs, Ws, P, win_t, win_h, win_w.
    """
    return _content_mask("nabla_build_mask", q, k, float(thr), sta, N, transpose, dense, out,
                         workspace, stream)


@_on_stream
def nabla_build_topk_mask(q: torch.Tensor, k: torch.Tensor, topk: int, sta: Optional[dict] = None,
                          N: int = BLOCK_N, *, transpose: bool = False, dense: bool = False,
                          out: Optional[Dict[str, torch.Tensor]] = None,
                          workspace: Optional[torch.Tensor] = None,
                          stream=None) -> Dict[str, torch.Tensor]:
    """Top-k selector: the topk largest reduced-map blocks of every row (ties kept
    together) [+ STA union]. Same outputs as nabla_build_mask."""
    return _content_mask("nabla_build_topk_mask", q, k, int(topk), sta, N, transpose, dense, out,
                         workspace, stream)


@_on_stream
def nabla_build_sta_mask(B: int, H: int, S: int, sta: dict, device, N: int = BLOCK_N, *,
                         transpose: bool = False, dense: bool = False,
                         out: Optional[Dict[str, torch.Tensor]] = None,
                         workspace: Optional[torch.Tensor] = None,
                         stream=None) -> Dict[str, torch.Tensor]:
    """The static STA window alone (section 2.2), as lists for every head."""
    device = torch.device(device)
    if sta is None:
        raise ValueError("the STA-only selector needs the sta window")
    _check_devices(device)
    res = _mask_outputs(B, H, S // N, device, transpose, dense, out)
    ws, size = _workspace(NABLA_OP_STA_MASK, B, H, S, 0, N, device, workspace)
    if stream is None:
        stream = torch.cuda.current_stream(device)
    st = load_library().nabla_build_sta_mask(
        B, H, S, N, _sta_ptr(sta), _ptr(res["kv_count"]), _ptr(res["kv_idx"]),
        _ptr(res.get("q_count")), _ptr(res.get("q_idx")), _ptr(res.get("dense_mask")), _ptr(ws),
        ws.numel(), ctypes.c_void_p(stream.cuda_stream))
    if st != NABLA_OK:
        raise NablaError(st, "nabla_build_sta_mask")
    return res


@_on_stream
def nabla_sparse_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          kv_count: torch.Tensor, kv_idx: torch.Tensor,
                          softmax_scale: Optional[float] = None, N: int = BLOCK_N, *,
                          o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          want_lse: bool = True, out_dtype: torch.dtype = torch.bfloat16,
                          frame_blocks: int = 0, workspace: Optional[torch.Tensor] = None,
                          stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Block-sparse attention forward (eq. (4) on the kept blocks).

    Returns (O, LSE fp32); O is bf16 or fp32 (``out_dtype``). ``frame_blocks``
    (blocks per latent frame, (Hs/P)*(Ws/P)) lets query blocks i and i + F share
    their K/V loads; results are identical with or without it."""
    _check_qkv("q", q)
    B, H, S, D = q.shape
    _check_qkv("k", k, q.shape)
    _check_qkv("v", v, q.shape)
    n = S // N
    _check_tensor("kv_count", kv_count, torch.int32, (B, H, n))
    _check_tensor("kv_idx", kv_idx, torch.int32, (B, H, n, n))
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
    if o is not None:
        _check_tensor("o", o, out_dtype, tuple(q.shape))
    if lse is not None:
        _check_tensor("lse", lse, torch.float32, (B, H, S))
    ws, size = _workspace(NABLA_OP_FWD, B, H, S, D, N, q.device, workspace)
    _check_devices(q.device, k=k, v=v, kv_count=kv_count, kv_idx=kv_idx, o=o, lse=lse)
    scale = (1.0 / math.sqrt(D)) if softmax_scale is None else float(softmax_scale)
    if o is None:
        o = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    o_dtype = NABLA_DTYPE_FP32 if out_dtype == torch.float32 else NABLA_DTYPE_BF16
    if want_lse and lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    st = load_library().nabla_sparse_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), B, H, S, D, N, _ptr(kv_count), _ptr(kv_idx), scale,
        int(frame_blocks), _ptr(o), o_dtype, _ptr(lse) if want_lse else None, _ptr(ws), ws.numel(), _stream(q, stream))
    if st != NABLA_OK:
        raise NablaError(st, "nabla_sparse_attn_fwd")
    return o, (lse if want_lse else None)


@_on_stream
def nabla_sparse_attn_fwd_static(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                 kv_count: torch.Tensor, kv_idx: torch.Tensor,
                                 softmax_scale: Optional[float] = None, N: int = BLOCK_N, *,
                                 o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                                 want_lse: bool = True, out_dtype: torch.dtype = torch.bfloat16,
                                 frame_blocks: int = 0,
                                 stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """nabla_sparse_attn_fwd without a workspace: the library's own device scratch
    is used (no allocation inside the call; outputs are allocated here only if
    not passed). Concurrent calls on one GPU race on that scratch."""
    _check_qkv("q", q)
    B, H, S, D = q.shape
    _check_qkv("k", k, q.shape)
    _check_qkv("v", v, q.shape)
    n = S // N
    _check_tensor("kv_count", kv_count, torch.int32, (B, H, n))
    _check_tensor("kv_idx", kv_idx, torch.int32, (B, H, n, n))
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
    if o is not None:
        _check_tensor("o", o, out_dtype, tuple(q.shape))
    if lse is not None:
        _check_tensor("lse", lse, torch.float32, (B, H, S))
    _check_devices(q.device, k=k, v=v, kv_count=kv_count, kv_idx=kv_idx, o=o, lse=lse)
    scale = (1.0 / math.sqrt(D)) if softmax_scale is None else float(softmax_scale)
    if o is None:
        o = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    o_dtype = NABLA_DTYPE_FP32 if out_dtype == torch.float32 else NABLA_DTYPE_BF16
    if want_lse and lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    st = load_library().nabla_sparse_attn_fwd_static(
        _ptr(q), _ptr(k), _ptr(v), B, H, S, D, N, _ptr(kv_count), _ptr(kv_idx), scale,
        int(frame_blocks), _ptr(o), o_dtype, _ptr(lse) if want_lse else None, _stream(q, stream))
    if st != NABLA_OK:
        raise NablaError(st, "nabla_sparse_attn_fwd_static")
    return o, (lse if want_lse else None)


@_on_stream
def nabla_sparse_attn_bwd(q, k, v, o, d_o, lse, kv_count, kv_idx, q_count, q_idx,
                          softmax_scale: Optional[float] = None, N: int = BLOCK_N, *,
                          dq=None, dk=None, dv=None, workspace=None,
                          stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Block-sparse attention backward with the mask held constant. Returns (dQ, dK, dV) bf16.

    ``o`` is the forward output, bf16 or fp32."""
    _check_qkv("q", q)
    B, H, S, D = q.shape
    for name, t in (("k", k), ("v", v), ("d_o", d_o)):
        _check_qkv(name, t, q.shape)
    _check_tensor("o", o, (torch.bfloat16, torch.float32), tuple(q.shape))
    o_dtype = NABLA_DTYPE_FP32 if o.dtype == torch.float32 else NABLA_DTYPE_BF16
    n = S // N
    for name, t, shp in (("kv_count", kv_count, (B, H, n)), ("kv_idx", kv_idx, (B, H, n, n)),
                         ("q_count", q_count, (B, H, n)), ("q_idx", q_idx, (B, H, n, n))):
        _check_tensor(name, t, torch.int32, shp)
    _check_tensor("lse", lse, torch.float32, (B, H, S))
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is not None:
            _check_qkv(name, t, q.shape)
    ws, size = _workspace(NABLA_OP_BWD, B, H, S, D, N, q.device, workspace)
    _check_devices(q.device, k=k, v=v, o=o, d_o=d_o, lse=lse, kv_count=kv_count, kv_idx=kv_idx,
                   q_count=q_count, q_idx=q_idx, dq=dq, dk=dk, dv=dv)
    scale = (1.0 / math.sqrt(D)) if softmax_scale is None else float(softmax_scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    st = load_library().nabla_sparse_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), o_dtype, _ptr(d_o), _ptr(lse), B, H, S, D, N, _ptr(kv_count),
        _ptr(kv_idx), _ptr(q_count), _ptr(q_idx), scale, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
        ws.numel(), _stream(q, stream))
    if st != NABLA_OK:
        raise NablaError(st, "nabla_sparse_attn_bwd")
    return dq, dk, dv


@_on_stream
def nabla_block_mass(q: torch.Tensor, k: torch.Tensor, lse: torch.Tensor,
                     softmax_scale: Optional[float] = None, N: int = BLOCK_N, *,
                     out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """True block mass of dense attention, M [B,H,n,n] fp32 (rows sum to 1).

    ``lse`` is the dense log-sum-exp [B,H,S] fp32, e.g. from nabla_sparse_attn_fwd
    over lists that keep every block."""
    _check_qkv("q", q)
    B, H, S, D = q.shape
    _check_qkv("k", k, q.shape)
    _check_tensor("lse", lse, torch.float32, (B, H, S))
    n = S // N
    if out is not None:
        _check_tensor("out", out, torch.float32, (B, H, n, n))
    _check_devices(q.device, k=k, lse=lse, out=out)
    if out is None:
        out = torch.empty((B, H, n, n), dtype=torch.float32, device=q.device)
    scale = (1.0 / math.sqrt(D)) if softmax_scale is None else float(softmax_scale)
    st = load_library().nabla_block_mass(_ptr(q), _ptr(k), _ptr(lse), B, H, S, D, N, scale, _ptr(out),
                                         _stream(q, stream))
    if st != NABLA_OK:
        raise NablaError(st, "nabla_block_mass")
    return out


@_on_stream
def nabla_mask_recall(mass: torch.Tensor, kv_count: torch.Tensor, kv_idx: torch.Tensor,
                      N: int = BLOCK_N, *, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per row: block mass inside the kept lists, and inside the best blocks at the same count."""
    if not isinstance(mass, torch.Tensor) or mass.dim() != 4:
        raise ValueError("mass must be a float32 tensor [B, H, n, n]")
    B, H, n, _ = mass.shape
    _check_tensor("mass", mass, torch.float32, (B, H, n, n))
    for name, t, shp in (("kv_count", kv_count, (B, H, n)), ("kv_idx", kv_idx, (B, H, n, n))):
        _check_tensor(name, t, torch.int32, shp)
    _check_devices(mass.device, kv_count=kv_count, kv_idx=kv_idx)
    recall = torch.empty((B, H, n), dtype=torch.float32, device=mass.device)
    best = torch.empty_like(recall)
    st = load_library().nabla_mask_recall(_ptr(mass), B, H, n * N, N, _ptr(kv_count), _ptr(kv_idx),
                                          _ptr(recall), _ptr(best), _stream(mass, stream))
    if st != NABLA_OK:
        raise NablaError(st, "nabla_mask_recall")
    return recall, best


@_on_stream
def nabla_check_lists(count: torch.Tensor, idx: torch.Tensor, N: int = BLOCK_N, *,
                      stream=None) -> int:
    """Number of rows whose list is malformed (count outside [0, n]; an entry outside
    [0, n) or not larger than its predecessor among the first count entries). Waits
    for the stream to reach the check (it returns a host integer)."""
    if not isinstance(count, torch.Tensor) or count.dim() != 3:
        raise ValueError("count must be an int32 tensor [B, H, n]")
    B, H, n = count.shape
    _check_tensor("count", count, torch.int32, (B, H, n))
    _check_tensor("idx", idx, torch.int32, (B, H, n, n))
    _check_devices(count.device, idx=idx)
    bad = torch.empty((), dtype=torch.int32, device=count.device)
    st = load_library().nabla_check_lists(_ptr(count), _ptr(idx), B, H, n * N, N, _ptr(bad),
                                          _stream(count, stream))
    if st != NABLA_OK:
        raise NablaError(st, "nabla_check_lists")
    return int(bad.item())


@_on_stream
def nabla_reorder_tokens(x: torch.Tensor, T: int, Hs: int, Ws: int, P: int, inverse: bool = False,
                         *, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Token reordering of section 3.1.1 (Figure 3) or its inverse, out of place.

    ``x`` is a contiguous CUDA tensor [..., T*Hs*Ws, F] (any dtype): the
    leading dimensions are items, each token's F features one row. Returns the
    tokens in block order (``inverse=False``) or back in raster order."""
    if not isinstance(x, torch.Tensor) or not x.is_contiguous() or x.dim() < 2:
        raise ValueError("x must be a contiguous tensor [..., T*Hs*Ws, F]")
    S = T * Hs * Ws
    if x.shape[-2] != S:
        raise ValueError(f"x has {x.shape[-2]} tokens, expected T*Hs*Ws = {S}")
    items = x.numel() // max(S * x.shape[-1], 1) if x.numel() else 0
    row_bytes = x.shape[-1] * x.element_size()
    if out is not None:
        _check_tensor("out", out, x.dtype, tuple(x.shape))
    _check_devices(x.device, out=out)
    if out is None:
        out = torch.empty_like(x)
    st = load_library().nabla_reorder_tokens(_ptr(x), _ptr(out), items, T, Hs, Ws, P, row_bytes,
                                             1 if inverse else 0, _stream(x, stream))
    if st != NABLA_OK:
        raise NablaError(st, "nabla_reorder_tokens")
    return out


__all__ = [
    "LIB_PATH", "BLOCK_N", "EXPORTED_SYMBOLS", "NablaError", "StaWindow", "load_library",
    "nabla_status_string", "nabla_workspace_size", "nabla_build_mask", "nabla_build_topk_mask",
    "nabla_build_sta_mask", "nabla_sparse_attn_fwd", "nabla_sparse_attn_fwd_static",
    "nabla_sparse_attn_bwd", "nabla_reorder_tokens", "nabla_block_mass", "nabla_mask_recall", "nabla_check_lists", "NABLA_OP_MASK", "NABLA_OP_FWD", "NABLA_OP_BWD", "NABLA_OP_STA_MASK",
]
