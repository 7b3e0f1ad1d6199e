"""The whole path can be captured in a HIP graph and replayed.

The library itself allocates, copies and synchronises nothing, so with every
output and workspace passed in, mask (with the transposed lists) + forward
(frame hint) + backward capture into one graph. The graph is replayed four
times on two alternating input sets copied into the captured buffers, with
eager work and a synchronisation between replays, and every replay must equal
the eager results for the same inputs bitwise -- which also shows that each
replay rebuilds the mask from the current inputs."""

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _nb():
    import block_sparse_attention_nabla_amd as nb
    nb.load_library()
    return nb


def test_path_replays_from_a_graph():
    nb = _nb()
    w = synth.get_workload("dit_small")
    thr = w.thr_for(0.80)
    F = (w.Hs // w.P) * (w.Ws // w.P)
    sets = []
    for step in (0, 1):
        x = synth.make_inputs(w, step=step)
        sets.append([x[c].cuda() for c in "qkv"] + [synth.make_dout(w, step=step).cuda()])
    q, k, v, do = (t.clone() for t in sets[0])  # the captured input buffers
    B, H, S, D = q.shape
    print(f"[graph] dit_small thr={thr:.4f} S={S} F={F}", flush=True)

    dev = q.device
    lists = nb.nabla_build_mask(q, k, thr, transpose=True)
    ws_mask = torch.empty(nb.nabla_workspace_size(nb.NABLA_OP_MASK, B, H, S, D), dtype=torch.uint8, device=dev)
    ws_fwd = torch.empty(nb.nabla_workspace_size(nb.NABLA_OP_FWD, B, H, S, D), dtype=torch.uint8, device=dev)
    ws_bwd = torch.empty(nb.nabla_workspace_size(nb.NABLA_OP_BWD, B, H, S, D), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def path():
        nb.nabla_build_mask(q, k, thr, transpose=True, out=lists, workspace=ws_mask)
        nb.nabla_sparse_attn_fwd(q, k, v, lists["kv_count"], lists["kv_idx"], o=o, lse=lse,
                                 frame_blocks=F, workspace=ws_fwd)
        nb.nabla_sparse_attn_bwd(q, k, v, o, do, lse, lists["kv_count"], lists["kv_idx"],
                                 lists["q_count"], lists["q_idx"], dq=dq, dk=dk, dv=dv,
                                 workspace=ws_bwd)

    def load(i):
        for dst, src in zip((q, k, v, do), sets[i]):
            dst.copy_(src)

    def snapshot():
        n = lists["kv_count"].shape[-1]
        out = {}
        for cnt, idx in (("kv_count", "kv_idx"), ("q_count", "q_idx")):
            valid = torch.arange(n, device=dev) < lists[cnt][..., None]
            out[cnt] = lists[cnt].clone()
            out[idx] = torch.where(valid, lists[idx], torch.full_like(lists[idx], -1))
        for name, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
            out[name] = t.clone()
        return out

    refs = []
    for i in (0, 1):
        load(i)
        path()
        torch.cuda.synchronize()
        refs.append(snapshot())
    assert not torch.equal(refs[0]["kv_count"], refs[1]["kv_count"])  # the two sets differ

    load(0)
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        path()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()

    scratch = torch.randn(1 << 20, device=dev)
    for rep, i in enumerate((0, 1, 0, 1)):
        load(i)
        graph.replay()
        scratch.mul_(0.5).add_(1.0)  # eager work between replays
        torch.cuda.synchronize()
        got = snapshot()
        for key, ref in refs[i].items():
            assert ref.shape == got[key].shape and torch.equal(ref.view(torch.uint8), got[key].view(torch.uint8)), \
                (rep, i, key)
        print(f"[graph] replay {rep} (input set {i}) equals the eager results", flush=True)
