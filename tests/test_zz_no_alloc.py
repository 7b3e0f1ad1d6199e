"""The allocation-free forward entry point (nabla_sparse_attn_fwd_static), called
through the C ABI with ctypes, against nabla_sparse_attn_fwd on the same inputs:
bitwise equal outputs on two calls in a row, the second with a smaller input (the
library-held scratch keeps the first call's contents), with and without the
frame hint; shapes beyond the scratch limit are rejected before any launch."""

import ctypes
import math

import pytest
import torch

pytestmark = pytest.mark.gpu

OK, WORKSPACE = 0, 3


def _nb():
    import block_sparse_attention_nabla_amd as nb
    nb.load_library()
    return nb


def _case(B, H, n, D, seed, thr):
    nb = _nb()
    g = torch.Generator().manual_seed(seed)
    S = 64 * n
    shp = (B, H, S, D)
    base = torch.randn((B, H, n, 1, D), generator=g)
    q = (torch.randn((B, H, n, 64, D), generator=g) + base).reshape(shp).bfloat16().cuda()
    k = (torch.randn((B, H, n, 64, D), generator=g) + base).reshape(shp).bfloat16().cuda()
    v = torch.randn(shp, generator=g).bfloat16().cuda()
    lists = nb.nabla_build_mask(q, k, thr)
    return q, k, v, lists


def _static_call(q, k, v, lists, frame_blocks, o_fp32):
    """The C entry point itself, with caller-allocated outputs and no workspace."""
    nb = _nb()
    B, H, S, D = q.shape
    o = torch.empty(q.shape, dtype=torch.float32 if o_fp32 else torch.bfloat16, device=q.device)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()
    st = nb.load_library().nabla_sparse_attn_fwd_static(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        B, H, S, D, 64, ctypes.c_void_p(lists["kv_count"].data_ptr()),
        ctypes.c_void_p(lists["kv_idx"].data_ptr()), 1.0 / math.sqrt(D), frame_blocks,
        ctypes.c_void_p(o.data_ptr()), 1 if o_fp32 else 0, ctypes.c_void_p(lse.data_ptr()),
        ctypes.c_void_p(stream.cuda_stream))
    assert st == OK, nb.nabla_status_string(st)
    return o, lse


@pytest.mark.parametrize("frame_blocks", [0, 4])
def test_static_forward_equals_workspace_forward_twice(frame_blocks):
    nb = _nb()
    # Second call smaller (fewer heads and blocks): stale scratch from the first
    # call must not leak into it.
    for (B, H, n, D, seed, thr, o_fp32) in ((2, 3, 96, 128, 1, 0.6, False), (1, 2, 40, 64, 2, 0.4, True)):
        print(f"[noalloc] B={B} H={H} n={n} D={D} frame_blocks={frame_blocks}", flush=True)
        q, k, v, lists = _case(B, H, n, D, seed, thr)
        o_ref, lse_ref = nb.nabla_sparse_attn_fwd(q, k, v, lists["kv_count"], lists["kv_idx"],
                                                  frame_blocks=frame_blocks,
                                                  out_dtype=torch.float32 if o_fp32 else torch.bfloat16)
        o, lse = _static_call(q, k, v, lists, frame_blocks, o_fp32)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16 if not o_fp32 else torch.int32),
                           o_ref.view(torch.int16 if not o_fp32 else torch.int32))
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32))


def test_static_forward_binding_and_limit():
    nb = _nb()
    q, k, v, lists = _case(1, 2, 64, 64, 3, 0.5)
    o_ref, lse_ref = nb.nabla_sparse_attn_fwd(q, k, v, lists["kv_count"], lists["kv_idx"])
    o, lse = nb.nabla_sparse_attn_fwd_static(q, k, v, lists["kv_count"], lists["kv_idx"])
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32))
    # 129 heads x 8192 blocks need more than the library-held scratch: rejected
    # before anything is launched (the small tensors are never touched).
    st = nb.load_library().nabla_sparse_attn_fwd_static(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        1, 129, 64 * 8192, 64, 64, ctypes.c_void_p(lists["kv_count"].data_ptr()),
        ctypes.c_void_p(lists["kv_idx"].data_ptr()), 0.125, 0, ctypes.c_void_p(o.data_ptr()), 0,
        None, None)
    assert st == WORKSPACE
