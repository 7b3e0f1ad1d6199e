"""Every entry point launches its kernels on the stream it is handed.

The whole path -- mask (with the transposed lists), forward with the frame
hint, backward, and token reordering with its inverse -- runs once on the
default stream and then on a side stream (default priority), both as the
current stream and passed explicitly while the default stream is current.
Results must be bitwise those of the default stream (every kernel is
deterministic), which fails if any launch lands on another stream before its
inputs are ready or after its outputs are read."""

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _nb():
    import block_sparse_attention_nabla_amd as nb
    nb.load_library()
    return nb


def _path(nb, w, q, k, v, do, tokens, thr, stream=None):
    F = (w.Hs // w.P) * (w.Ws // w.P)
    m = nb.nabla_build_mask(q, k, thr, transpose=True, stream=stream)
    o, lse = nb.nabla_sparse_attn_fwd(q, k, v, m["kv_count"], m["kv_idx"], frame_blocks=F,
                                      stream=stream)
    dq, dk, dv = nb.nabla_sparse_attn_bwd(q, k, v, o, do, lse, m["kv_count"], m["kv_idx"],
                                          m["q_count"], m["q_idx"], stream=stream)
    blocks = nb.nabla_reorder_tokens(tokens, w.T, w.Hs, w.Ws, w.P, stream=stream)
    raster = nb.nabla_reorder_tokens(blocks, w.T, w.Hs, w.Ws, w.P, inverse=True, stream=stream)
    return {"kv_count": m["kv_count"], "kv_idx": m["kv_idx"], "q_count": m["q_count"],
            "q_idx": m["q_idx"], "o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv,
            "blocks": blocks, "raster": raster}


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return a.shape == b.shape and torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def _check(ref, got):
    n = ref["kv_count"].shape[-1]
    for cnt, idx in (("kv_count", "kv_idx"), ("q_count", "q_idx")):
        assert torch.equal(ref[cnt], got[cnt]), cnt
        valid = torch.arange(n, device=ref[cnt].device) < ref[cnt][..., None]  # defined entries
        assert torch.equal(ref[idx][valid], got[idx][valid]), idx
    for key in ("o", "lse", "dq", "dk", "dv", "blocks", "raster"):
        assert _same(ref[key], got[key]), key


def test_side_stream_gives_default_stream_results():
    nb = _nb()
    w = synth.get_workload("dit_small")
    thr = w.thr_for(0.80)
    x = synth.make_inputs(w)
    q, k, v = (x[c].cuda() for c in "qkv")
    do = synth.make_dout(w).cuda()
    g = torch.Generator().manual_seed(5)
    tokens = torch.randn((2, w.T * w.Hs * w.Ws, 96), generator=g).bfloat16().cuda()
    print(f"[streams] dit_small thr={thr:.4f} S={w.T * w.Hs * w.Ws}", flush=True)

    ref = _path(nb, w, q, k, v, do, tokens, thr)
    torch.cuda.synchronize()
    assert torch.equal(ref["raster"], tokens)

    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = _path(nb, w, q, k, v, do, tokens, thr)
    side.synchronize()
    _check(ref, got)

    # Explicit stream argument while the default stream is current: outputs are
    # allocated on the current stream, so the side stream waits for it first.
    side.wait_stream(torch.cuda.current_stream())
    got2 = _path(nb, w, q, k, v, do, tokens, thr, stream=side)
    side.synchronize()
    _check(ref, got2)
