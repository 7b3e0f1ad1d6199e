"""The Python binding checks every tensor it hands to the C ABI -- dtype, shape,
contiguity and device -- and raises ValueError before anything is launched.
Runs without a GPU: shape and dtype checks come first, so CPU tensors reach each
of them, and correct CPU tensors are then rejected for not being on a HIP device."""

import os

import pytest
import torch

import block_sparse_attention_nabla_amd as nb

B, H, S, D = 1, 2, 256, 64
n = S // 64


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(nb.LIB_PATH):
        pytest.fail("libnabla.so is not built (run python -m block_sparse_attention_nabla_amd.build)")
    return nb.load_library()


def _qkv():
    return [torch.zeros((B, H, S, D), dtype=torch.bfloat16) for _ in range(3)]


def _lists():
    return (torch.zeros((B, H, n), dtype=torch.int32), torch.zeros((B, H, n, n), dtype=torch.int32))


def _raises(match, fn, *args, **kwargs):
    with pytest.raises(ValueError, match=match):
        fn(*args, **kwargs)


def test_forward_arguments():
    q, k, v = _qkv()
    cnt, idx = _lists()
    _raises("k has shape", nb.nabla_sparse_attn_fwd, q, k[:, :1].contiguous(), v, cnt, idx)
    _raises("v must be a contiguous bfloat16", nb.nabla_sparse_attn_fwd, q, k, v.float(), cnt, idx)
    _raises("kv_count has dtype", nb.nabla_sparse_attn_fwd, q, k, v, cnt.long(), idx)
    _raises("kv_idx has shape", nb.nabla_sparse_attn_fwd, q, k, v, cnt, idx[..., :3])
    _raises("kv_idx must be contiguous", nb.nabla_sparse_attn_fwd, q, k, v, cnt,
            idx.transpose(-1, -2))
    _raises("lse has shape", nb.nabla_sparse_attn_fwd, q, k, v, cnt, idx,
            lse=torch.zeros((B, H, S - 1), dtype=torch.float32))
    _raises("lse has dtype", nb.nabla_sparse_attn_fwd, q, k, v, cnt, idx,
            lse=torch.zeros((B, H, S), dtype=torch.float64))
    _raises("o has dtype", nb.nabla_sparse_attn_fwd, q, k, v, cnt, idx, o=torch.zeros_like(q).float())
    _raises("o has shape", nb.nabla_sparse_attn_fwd, q, k, v, cnt, idx, o=q[:, :1].contiguous())
    _raises("workspace holds", nb.nabla_sparse_attn_fwd, q, k, v, cnt, idx,
            workspace=torch.zeros(4, dtype=torch.uint8))
    _raises("workspace has dtype", nb.nabla_sparse_attn_fwd, q, k, v, cnt, idx,
            workspace=torch.zeros(1 << 20, dtype=torch.float32))
    # everything well formed, but on the host
    _raises("HIP", nb.nabla_sparse_attn_fwd, q, k, v, cnt, idx)


def test_backward_arguments():
    q, k, v = _qkv()
    cnt, idx = _lists()
    lse = torch.zeros((B, H, S), dtype=torch.float32)
    args = [q, k, v, q.clone(), q.clone(), lse, cnt, idx, cnt.clone(), idx.clone()]
    bad_dq = torch.zeros((B, H, S, D + 1), dtype=torch.bfloat16)
    _raises("dq has shape", nb.nabla_sparse_attn_bwd, *args, dq=bad_dq)
    _raises("dv must be a contiguous bfloat16", nb.nabla_sparse_attn_bwd, *args,
            dv=torch.zeros_like(q).float())
    bad = list(args)
    bad[5] = lse[..., :-1]
    _raises("lse has shape", nb.nabla_sparse_attn_bwd, *bad)
    bad = list(args)
    bad[3] = q.half()
    _raises("o has dtype", nb.nabla_sparse_attn_bwd, *bad)
    bad = list(args)
    bad[9] = idx.float()
    _raises("q_idx has dtype", nb.nabla_sparse_attn_bwd, *bad)
    _raises("HIP", nb.nabla_sparse_attn_bwd, *args)


def test_mask_arguments():
    q, k, _ = _qkv()
    _raises("k has shape", nb.nabla_build_mask, q, k[..., :32].contiguous(), 0.5)
    out = {"kv_count": torch.zeros((B, H, n), dtype=torch.int64)}
    _raises("kv_count", nb.nabla_build_mask, q, k, 0.5, out=out)
    out = {"dense_mask": torch.zeros((B, H, n, n + 1), dtype=torch.uint8)}
    _raises("dense_mask", nb.nabla_build_mask, q, k, 0.5, dense=True, out=out)
    _raises("workspace holds", nb.nabla_build_mask, q, k, 0.5, workspace=torch.zeros(8, dtype=torch.uint8))
    _raises("HIP", nb.nabla_build_mask, q, k, 0.5)
    _raises("HIP", nb.nabla_build_topk_mask, q, k, 3)
    sta = {"T": 1, "Hs": 16, "Ws": 16, "P": 8, "win_t": 1, "win_h": 8, "win_w": 8}
    _raises("HIP", nb.nabla_build_sta_mask, B, H, S, sta, "cpu")


def test_diagnostic_and_reorder_arguments():
    q, k, _ = _qkv()
    lse = torch.zeros((B, H, S), dtype=torch.float32)
    _raises("out has shape", nb.nabla_block_mass, q, k, lse, out=torch.zeros((B, H, n, n - 1)))
    _raises("lse has dtype", nb.nabla_block_mass, q, k, lse.double())
    _raises("HIP", nb.nabla_block_mass, q, k, lse)
    mass = torch.zeros((B, H, n, n), dtype=torch.float32)
    cnt, idx = _lists()
    _raises("kv_idx has shape", nb.nabla_mask_recall, mass, cnt, idx[:, :1].contiguous())
    _raises("mass has dtype", nb.nabla_mask_recall, mass.double(), cnt, idx)
    _raises("HIP", nb.nabla_mask_recall, mass, cnt, idx)
    x = torch.zeros((1, 4 * 16 * 16, 32), dtype=torch.bfloat16)
    _raises("out has shape", nb.nabla_reorder_tokens, x, 4, 16, 16, 8, out=x[:, :-1].contiguous())
    _raises("HIP", nb.nabla_reorder_tokens, x, 4, 16, 16, 8)


def test_check_lists_arguments():
    cnt, idx = _lists()
    _raises("count must be", nb.nabla_check_lists, cnt.reshape(-1), idx)
    _raises("count has dtype", nb.nabla_check_lists, cnt.long(), idx)
    _raises("idx has shape", nb.nabla_check_lists, cnt, idx[..., :1].contiguous())
    _raises("idx has dtype", nb.nabla_check_lists, cnt, idx.float())
    _raises("CUDA", nb.nabla_check_lists, cnt, idx)
