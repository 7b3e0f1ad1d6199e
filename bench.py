"""Benchmark of the NABLA hot path on one MI355X.

One step = the whole forward hot path on the Wan 2.1 14B-like 720p layer
(B=1, H=40, S=80640, D=128, N=64; 1260 blocks per head) at 90% block sparsity:
    nabla_build_mask  (pool Q/K, reduced logits, CDF selection, compaction)
    nabla_sparse_attn_fwd  (longest-first order + block-sparse flash forward)
on inputs already resident in HBM. The metric is effective TFLOP/s on kept
blocks: 4*N*N*D FLOP per kept (query block, key block) pair, divided by the
step time. Also reported: the forward kernel's own TFLOP/s against the bf16
MFMA peak (roofline), the speedup over the same kernel run dense, the mask
stage's HBM GB/s, and the CPU oracle timed on a bounded sample of the same
workload. Under "configs": the other operating point of the layer (80%), the
layer on the literal std-3 input recipe, and the smaller workloads (the tiny
threshold sweep, the ~80%-sparse DiT-small layer and its STA union), each with
the same kernels' dense time, speedup, linearity and load-balance efficiency
(the time the dense per-pair rate predicts for the kept pairs over the measured
time), and the CPU oracle timed over each whole small workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--sparsity S] [--no-cpu-baseline]
Prints ONE JSON line on stdout; progress goes to stderr.

HBM traffic of the forward kernel (roofline "traffic"): run twice under
rocprofv3 with the counters FETCH_SIZE and WRITE_SIZE,
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR -o fetch -- \
        python bench.py --steps 1 --warmup 1 --no-dense --no-cpu-baseline --traffic-calibration
(and the same with WRITE_SIZE), then
    python bench.py --summarize-traffic DIR/fetch_counter_collection.csv DIR/write_counter_collection.csv
which scales each counter by what it reads for a plain 1 GiB copy kernel run
in the same process and records the result, keyed to the forward kernel's
source, for later bench runs. With --traffic-kernel attn_fwd_kernel (counters
taken with --no-pairs) it prints the one-block kernel's figures instead and
records nothing.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s on kept blocks (% bf16 MFMA peak) + speedup vs dense at ~90% sparsity"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
# The forward kernel that bench.py times: the paired kernel when the frame hint is
# given (the default), the one-block kernel with --no-pairs.
FWD_KERNEL = "attn_fwd_pair_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_wan14b_720p_traffic.json")
# Everything the forward kernel's code and work order come from: counters taken
# on other sources are not reported.
FWD_SOURCES = [os.path.join(ROOT, "block_sparse_attention_nabla_amd", "csrc", f)
               for f in ("attn_fwd.hip", "kernels.h", "common.h", "schedule.hip")]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(launch_flops: float):
    """HBM bytes per forward launch from committed rocprofv3 counters, if they
    were taken on the current forward kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != source_hash(FWD_SOURCES):
        return None
    return t.get("bytes_per_launch")


CALIB_BYTES = 1 << 30  # copy-kernel calibration: read and write 1 GiB


def summarize_traffic(fetch_csv: str, write_csv: str, kernel: str = FWD_KERNEL) -> dict:
    """Per-launch HBM bytes of a forward kernel from two rocprofv3 counter CSVs.
    Only the figures of the kernel bench.py times (FWD_KERNEL) are recorded."""
    import csv

    def per_kernel(path, counter):
        out = {"fwd": [], "copy": []}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            kb = float(r["Counter_Value"])
            if kernel + "<" in r["Kernel_Name"]:
                out["fwd"].append(kb)
            elif "elementwise" in r["Kernel_Name"] and int(r["Grid_Size"]) > (1 << 20):
                out["copy"].append(kb)
        return out

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    wr = per_kernel(write_csv, "WRITE_SIZE")
    if not (f["fwd"] and f["copy"] and wr["fwd"] and wr["copy"]):
        raise SystemExit("counter CSVs lack forward or calibration-copy dispatches")
    f_scale = (CALIB_BYTES / 1024.0) / max(f["copy"])
    w_scale = (CALIB_BYTES / 1024.0) / max(wr["copy"])
    fetch_b = sum(f["fwd"]) / len(f["fwd"]) * 1024.0 * f_scale
    write_b = sum(wr["fwd"]) / len(wr["fwd"]) * 1024.0 * w_scale
    res = {
        "kernel": kernel,
        "workload": "wan14b_720p at 90% block sparsity",
        "fetch_bytes_per_launch": fetch_b,
        "write_bytes_per_launch": write_b,
        "bytes_per_launch": fetch_b + write_b,
        "calibration": {"copy_bytes": CALIB_BYTES, "fetch_scale": f_scale, "write_scale": w_scale,
                        "raw_copy_fetch_kb": max(f["copy"]), "raw_copy_write_kb": max(wr["copy"])},
        "launches": {"fetch": len(f["fwd"]), "write": len(wr["fwd"])},
        "kernel_source_sha256_16": source_hash(FWD_SOURCES),
    }
    if kernel != FWD_KERNEL:
        return res
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(res, fh, indent=2)
    return res


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x, thr: float, heads: int = 2, gpu_dense_mask=None) -> dict:
    """The oracle on a bounded sample of the same workload: the whole hot path
    (mask, then the masked forward over every query block) for the first
    `heads` heads; the rate is kept-block FLOP of the sample over its time.
    With the GPU's dense mask of those heads, also the mask parity counts
    (blocks in the 1e-5 band of thr, mismatches, unexplained mismatches)."""
    import oracle

    q = x["q"].reshape(-1, w.S, w.D)[:heads].float()
    k = x["k"].reshape(-1, w.S, w.D)[:heads].float()
    v = x["v"].reshape(-1, w.S, w.D)[:heads].float()
    t0 = time.perf_counter()
    m = oracle.build_mask(q, k, w.N, thr)
    t_mask = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.attn_fwd(q, k, v, m["mask"], w.N)
    t_fwd = time.perf_counter() - t0
    kept = int(m["mask"].sum())
    flops = kept * 4.0 * w.N * w.N * w.D
    parity = None
    if gpu_dense_mask is not None:
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from parity import compare_masks
        parity = compare_masks(gpu_dense_mask[:heads], m, thr)
    return {"value": flops / (t_mask + t_fwd) / 1e12, "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "cpu": cpu_model(), "kind": "oracle",
            "mask_parity_sample": parity,
            "sample": (f"heads 0..{heads - 1} of {w.B * w.H}: mask ({t_mask:.1f} s) and forward over all "
                       f"{w.n} query blocks per head ({kept} kept blocks, {t_fwd:.1f} s); "
                       f"fp64 C + OpenMP"),
            "seconds": round(t_mask + t_fwd, 2)}


def recall_summary(nb, mass, lists) -> dict:
    """Mask fidelity of block lists: mass of dense attention inside the kept blocks,
    against the best blocks at the same per-row count (per-row means and tails)."""
    import torch
    rec, best = nb.nabla_mask_recall(mass, lists["kv_count"], lists["kv_idx"])
    r = rec.reshape(-1).double()
    b = best.reshape(-1).double()
    return {
        "mean_recall": round(float(r.mean()), 5),
        "mean_best_recall": round(float(b.mean()), 5),
        "recall_p01": round(float(torch.quantile(r.float().cpu(), 0.01)), 5),
        "min_recall": round(float(r.min()), 5),
        "mean_gap_to_best": round(float((b - r).mean()), 5),
    }


def selector_bench(w, q, k, v, lists, ws_mask, ws_fwd, o, lse, stream, iters: int,
                   topk: int, sta_win, mass=None, frame_blocks: int = 0) -> dict:
    """The variant selectors on the same layer: Top-k blocks (k = topk) and the
    static STA window alone, each followed by the same forward kernel. With the
    dense block mass, also the fidelity of each selector's lists."""
    import torch
    import block_sparse_attention_nabla_amd as nb
    B, H, S, D, n = w.B, w.H, w.S, w.D, w.n
    sta = dict(T=w.T, Hs=w.Hs, Ws=w.Ws, P=w.P, win_t=sta_win[0], win_h=sta_win[1], win_w=sta_win[2])
    ws_sta = torch.empty(nb.nabla_workspace_size(nb.NABLA_OP_STA_MASK, B, H, S, D), dtype=torch.uint8,
                         device=q.device)
    makers = {
        "topk": lambda: nb.nabla_build_topk_mask(q, k, topk, out=lists, workspace=ws_mask, stream=stream),
        "sta_only": lambda: nb.nabla_build_sta_mask(B, H, S, sta, q.device, out=lists, workspace=ws_sta,
                                                    stream=stream),
    }
    res = {}
    for name, make in makers.items():
        def fwd():
            nb.nabla_sparse_attn_fwd(q, k, v, lists["kv_count"], lists["kv_idx"], o=o, lse=lse,
                                     workspace=ws_fwd, stream=stream, frame_blocks=frame_blocks)
        make()
        fwd()
        torch.cuda.synchronize()
        kept = int(lists["kv_count"].sum())
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(iters)]
        for i in range(iters):
            ev[i][0].record(stream)
            make()
            ev[i][1].record(stream)
            fwd()
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        mask_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / iters
        fwd_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / iters
        flops = kept * 4.0 * w.N * w.N * D
        res[name] = {
            "selector": f"top-{topk} blocks per row" if name == "topk" else f"STA{tuple(sta_win)} window alone",
            "block_sparsity": round(1.0 - kept / (B * H * n * n), 5),
            "mask_ms": round(mask_ms, 4), "forward_ms": round(fwd_ms, 4),
            "forward_tflops": round(flops / (fwd_ms * 1e-3) / 1e12, 2),
        }
        if mass is not None:
            res[name]["fidelity"] = recall_summary(nb, mass, lists)
        log(f"selector {name}: {res[name]}")
    return res


def reorder_bench(w, dev, stream, iters: int) -> dict:
    """Token reordering and its inverse on the workload's hidden states [B, S, H*D] bf16.

    A pure permutation: the algorithmic traffic is one read and one write of the tensor."""
    import torch
    import block_sparse_attention_nabla_amd as nb
    shape = (w.B, w.S, w.H * w.D)
    g = torch.Generator(device=dev).manual_seed(7)
    x = torch.randn(shape, generator=g, device=dev, dtype=torch.float32).bfloat16()
    y = torch.empty_like(x)
    z = torch.empty_like(x)
    for _ in range(2):
        nb.nabla_reorder_tokens(x, w.T, w.Hs, w.Ws, w.P, out=y, stream=stream)
        nb.nabla_reorder_tokens(y, w.T, w.Hs, w.Ws, w.P, inverse=True, out=z, stream=stream)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(stream)
    for _ in range(iters):
        nb.nabla_reorder_tokens(x, w.T, w.Hs, w.Ws, w.P, out=y, stream=stream)
    ev[1].record(stream)
    for _ in range(iters):
        nb.nabla_reorder_tokens(y, w.T, w.Hs, w.Ws, w.P, inverse=True, out=z, stream=stream)
    ev[2].record(stream)
    torch.cuda.synchronize()
    if not torch.equal(z.view(torch.int16), x.view(torch.int16)):
        raise RuntimeError("token reordering round trip is not the identity")
    nbytes = 2 * x.numel() * x.element_size()
    fwd_ms = ev[0].elapsed_time(ev[1]) / iters
    inv_ms = ev[1].elapsed_time(ev[2]) / iters
    fwd_gbps = nbytes / (fwd_ms * 1e-3) / 1e9
    inv_gbps = nbytes / (inv_ms * 1e-3) / 1e9
    log(f"token reordering {shape} bf16: forward {fwd_ms * 1e3:.1f} us ({fwd_gbps:.0f} GB/s), "
        f"inverse {inv_ms * 1e3:.1f} us ({inv_gbps:.0f} GB/s)")
    return {
        "kernel": "reorder_kernel",
        "shape": list(shape), "dtype": "bf16", "patch": w.P,
        "algorithmic_bytes_per_launch": nbytes,
        "fwd_ms": round(fwd_ms, 4), "inv_ms": round(inv_ms, 4),
        "fwd_gbps": round(fwd_gbps, 1), "inv_gbps": round(inv_gbps, 1),
        "bound": "hbm", "peak_gbps": PEAK_HBM_GBPS,
        "frac": round(max(fwd_gbps, inv_gbps) / PEAK_HBM_GBPS, 4),
    }


def train_step(args, dev, stream) -> dict:
    """Mask + forward + backward on the 2B-DiT training shape (B=2, H=16, S=61440,
    D=128; ~85% block sparsity). Every step rebuilds the mask from fresh Q/K
    (generated on the GPU from the same recipe, one seed per step)."""
    import torch
    import block_sparse_attention_nabla_amd as nb
    import synth

    w = synth.get_workload("dit2b_train")
    thr = w.thr_for(0.85)
    fb = 0 if args.no_pairs else (w.Hs // w.P) * (w.Ws // w.P)
    B, H, S, D, n = w.B, w.H, w.S, w.D, w.n
    steps = max(1, args.train_steps)
    t0 = time.time()
    sets = [synth.make_inputs(w, step=s + 1, device=dev) for s in range(steps + 1)]
    d_o = synth.make_dout(w, device=dev)
    log(f"train: {steps + 1} fresh input sets generated on the GPU in {time.time() - t0:.1f} s")
    lists = {"kv_count": torch.empty((B, H, n), dtype=torch.int32, device=dev),
             "kv_idx": torch.empty((B, H, n, n), dtype=torch.int32, device=dev),
             "q_count": torch.empty((B, H, n), dtype=torch.int32, device=dev),
             "q_idx": torch.empty((B, H, n, n), dtype=torch.int32, device=dev)}
    ws = {op: torch.empty(nb.nabla_workspace_size(op, B, H, S, D), dtype=torch.uint8, device=dev)
          for op in (nb.NABLA_OP_MASK, nb.NABLA_OP_FWD, nb.NABLA_OP_BWD)}
    o = torch.empty((B, H, S, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(o) for _ in range(3))

    def one(x, ev=None):
        if ev: ev[0].record(stream)
        nb.nabla_build_mask(x["q"], x["k"], thr, transpose=True, out=lists,
                            workspace=ws[nb.NABLA_OP_MASK], stream=stream)
        if ev: ev[1].record(stream)
        nb.nabla_sparse_attn_fwd(x["q"], x["k"], x["v"], lists["kv_count"], lists["kv_idx"], o=o,
                                 lse=lse, workspace=ws[nb.NABLA_OP_FWD], stream=stream,
                                 frame_blocks=fb)
        if ev: ev[2].record(stream)
        nb.nabla_sparse_attn_bwd(x["q"], x["k"], x["v"], o, d_o, lse, lists["kv_count"],
                                 lists["kv_idx"], lists["q_count"], lists["q_idx"], dq=dq, dk=dk,
                                 dv=dv, workspace=ws[nb.NABLA_OP_BWD], stream=stream)
        if ev: ev[3].record(stream)

    one(sets[0])  # warm-up
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    kept = []
    t_start = time.perf_counter()
    for i in range(steps):
        one(sets[i + 1], evs[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t_start) * 1e3 / steps
    kept_last = int(lists["kv_count"].sum())
    mask_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    fwd_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    bwd_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / steps
    fpk = 4.0 * w.N * w.N * D
    # Mask sparsity at the calibrated thr on fresh Q/K sets (one seed per step).
    del sets
    per_step = []
    for s_ in range(max(0, args.train_sparsity_steps)):
        xs = synth.make_inputs(w, step=100 + s_, device=dev)
        nb.nabla_build_mask(xs["q"], xs["k"], thr, out=lists, workspace=ws[nb.NABLA_OP_MASK],
                            stream=stream)
        per_step.append(round(1.0 - int(lists["kv_count"].sum()) / (B * H * n * n), 5))
        del xs
    res = {
        "workload": f"{w.name}: {w.description}",
        "thr": round(thr, 6),
        "block_sparsity_last_step": round(1.0 - kept_last / (B * H * n * n), 5),
        "ms_per_step": round(wall, 3),
        "mask_ms": round(mask_ms, 3),
        "forward_ms": round(fwd_ms, 3),
        "backward_ms": round(bwd_ms, 3),
        "forward_tflops": round(kept_last * fpk / (fwd_ms * 1e-3) / 1e12, 1),
        "backward_tflops": round(2.5 * kept_last * fpk / (bwd_ms * 1e-3) / 1e12, 1),
        "step_tflops": round(3.5 * kept_last * fpk / (wall * 1e-3) / 1e12, 1),
        "flop_model": "forward 4*N*N*D, backward 10*N*N*D per kept block pair",
        "frame_blocks": fb,
        "block_sparsity_per_fresh_step": per_step,
    }
    log(f"train: {res}")
    return res


def _time_calls(fn, stream, iters: int) -> float:
    """Average milliseconds of fn() over `iters` calls, HIP events on `stream`."""
    import torch
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def sparse_point(nb, w, q, k, v, thr, stream, iters, fb, dense_ms=None, sta=None, x_host=None,
                 ws=None, oracle_full=False) -> dict:
    """Mask + forward timings of one (workload, threshold) on the GPU; with the dense
    forward time of the same kernel, the speedup, linearity and the load-balance
    efficiency (the sparse time the dense per-pair rate predicts, over the measured
    time); optionally the CPU oracle over the whole workload (mask + forward)."""
    import torch
    B, H, S, D, n = w.B, w.H, w.S, w.D, w.n
    dev = q.device
    if ws is None:
        ws = {op: torch.empty(nb.nabla_workspace_size(op, B, H, S, D), dtype=torch.uint8, device=dev)
              for op in (nb.NABLA_OP_MASK, nb.NABLA_OP_FWD)}
    lists = {"kv_count": torch.empty((B, H, n), dtype=torch.int32, device=dev),
             "kv_idx": torch.empty((B, H, n, n), dtype=torch.int32, device=dev)}
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)

    def mask():
        nb.nabla_build_mask(q, k, thr, sta, out=lists, workspace=ws[nb.NABLA_OP_MASK], stream=stream)

    def fwd():
        nb.nabla_sparse_attn_fwd(q, k, v, lists["kv_count"], lists["kv_idx"], o=o, lse=lse,
                                 workspace=ws[nb.NABLA_OP_FWD], stream=stream, frame_blocks=fb)
    mask_ms = _time_calls(mask, stream, iters)
    mask()
    fwd_ms = _time_calls(fwd, stream, iters)
    counts = lists["kv_count"].reshape(-1)
    kept = int(counts.sum())
    density = kept / (B * H * n * n)
    flops = kept * 4.0 * w.N * w.N * D
    res = {"thr": round(thr, 6), "block_sparsity": round(1.0 - density, 5),
           "kept_per_row": {"min": int(counts.min()), "mean": round(kept / (B * H * n), 1),
                            "max": int(counts.max())},
           "mask_ms": round(mask_ms, 4), "forward_ms": round(fwd_ms, 4),
           "forward_tflops": round(flops / (fwd_ms * 1e-3) / 1e12, 2),
           "frac_bf16_peak": round(flops / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    if dense_ms is not None:
        speedup = dense_ms / fwd_ms
        res.update(dense_forward_ms=round(dense_ms, 4), speedup_vs_dense_forward=round(speedup, 3),
                   speedup_vs_dense_with_mask=round(dense_ms / (mask_ms + fwd_ms), 3),
                   linearity=round(speedup * density, 3),
                   load_balance_efficiency=round(density * dense_ms / fwd_ms, 3))
    if oracle_full and x_host is not None:
        import oracle
        qh, kh, vh = (x_host[key].reshape(-1, S, D).float() for key in ("q", "k", "v"))
        t0 = time.perf_counter()
        m = oracle.build_mask(qh, kh, w.N, thr, sta=sta)
        t_mask = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.attn_fwd(qh, kh, vh, m["mask"], w.N)
        t_fwd = time.perf_counter() - t0
        okept = int(m["mask"].sum())
        res["cpu_oracle_full"] = {
            "seconds": round(t_mask + t_fwd, 3), "mask_s": round(t_mask, 3), "forward_s": round(t_fwd, 3),
            "tflops": round(okept * 4.0 * w.N * w.N * D / (t_mask + t_fwd) / 1e12, 4),
            "cores": oracle.num_threads(), "kind": "oracle", "kept_blocks": okept,
            "gpu_speedup": round((t_mask + t_fwd) * 1e3 / (mask_ms + fwd_ms), 1)}
    return res


def dense_sdpa_ms(q, k, v, stream, iters):
    """torch.nn.functional.scaled_dot_product_attention on the same bf16 Q, K, V with
    the flash backend forced (no fallback to the unfused math path); None if that
    backend is unavailable for the shape."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    try:
        with torch.cuda.stream(stream), sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            F.scaled_dot_product_attention(q, k, v)
            torch.cuda.synchronize()
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(iters)]
            for e in ev:
                e[0].record(stream)
                F.scaled_dot_product_attention(q, k, v)
                e[1].record(stream)
            torch.cuda.synchronize()
    except RuntimeError as exc:
        log(f"torch SDPA flash backend unavailable: {exc}")
        return None
    ms = sum(e[0].elapsed_time(e[1]) for e in ev) / iters
    log(f"torch SDPA (flash) dense forward {ms:.2f} ms")
    return ms


def dense_forward_ms(nb, w, q, k, v, stream, iters, fb) -> float:
    """The same forward kernel with every block kept (thr >= 1 lists)."""
    import torch
    B, H, S, D, n = w.B, w.H, w.S, w.D, w.n
    dev = q.device
    lists = {"kv_count": torch.empty((B, H, n), dtype=torch.int32, device=dev),
             "kv_idx": torch.empty((B, H, n, n), dtype=torch.int32, device=dev)}
    nb.nabla_build_mask(q, k, 1.0, out=lists, stream=stream)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    ws = torch.empty(nb.nabla_workspace_size(nb.NABLA_OP_FWD, B, H, S, D), dtype=torch.uint8, device=dev)
    return _time_calls(lambda: nb.nabla_sparse_attn_fwd(q, k, v, lists["kv_count"], lists["kv_idx"], o=o,
                                                        lse=lse, workspace=ws, stream=stream,
                                                        frame_blocks=fb), stream, iters)


def small_configs(nb, dev, stream, args) -> dict:
    """The smaller workloads on the GPU (mask + forward, dense comparison, load-balance
    efficiency) with the CPU oracle timed over each whole workload: the threshold
    sweep of the tiny check, the ~80%-sparse DiT-small layer and the same layer
    with the STA(11,24,24) union."""
    import synth
    out = {}
    for name in ("tiny", "dit_small", "dit_small_sta"):
        w = synth.get_workload(name)
        x = synth.make_inputs(w)
        q, k, v = (x[key].bfloat16().to(dev) for key in ("q", "k", "v"))
        fb = 0 if args.no_pairs else (w.Hs // w.P) * (w.Ws // w.P)
        dense_ms = dense_forward_ms(nb, w, q, k, v, stream, args.config_iters, fb)
        xh = {key: x[key].bfloat16() for key in ("q", "k", "v")}
        thrs = w.thresholds()
        pts = {}
        for thr in thrs:
            pts[f"thr={thr:.4f}"] = sparse_point(nb, w, q, k, v, thr, stream, args.config_iters, fb,
                                                 dense_ms=dense_ms, sta=w.sta_struct(), x_host=xh,
                                                 oracle_full=not args.no_cpu_baseline)
        out[name] = {"workload": f"{name}: {w.description}", "frame_blocks": fb, "points": pts}
        log(f"config {name}: {out[name]}")
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan14b_720p")
    ap.add_argument("--sparsity", type=float, default=0.90)
    ap.add_argument("--dense-iters", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense comparison run")
    ap.add_argument("--traffic-calibration", action="store_true",
                    help="also run a plain 1 GiB copy kernel (counter calibration)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--traffic-kernel", default=FWD_KERNEL,
                    help="kernel whose counters --summarize-traffic reads (attn_fwd_kernel: print only)")
    ap.add_argument("--no-train", action="store_true",
                    help="skip the training-step figures (2B-DiT shape, forward + backward)")
    ap.add_argument("--train-steps", type=int, default=4)
    ap.add_argument("--train-sparsity-steps", type=int, default=10,
                    help="fresh Q/K sets whose mask sparsity is reported at the calibrated thr")
    ap.add_argument("--cold-iters", type=int, default=5,
                    help="mask + forward calls timed after a cache flush (0 = skip)")
    ap.add_argument("--no-pairs", action="store_true",
                    help="no frame hint: one query block per forward workgroup")
    ap.add_argument("--no-fidelity", action="store_true",
                    help="skip the mask-fidelity diagnostic (needs the dense run)")
    ap.add_argument("--no-selectors", action="store_true",
                    help="skip the Top-k and STA-only selector measurement")
    ap.add_argument("--no-reorder", action="store_true",
                    help="skip the token reordering measurement")
    ap.add_argument("--reorder-iters", type=int, default=10)
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other operating points and workloads (720p at 80%%, literal "
                         "std-3 inputs, tiny / dit_small / dit_small_sta with the full CPU oracle)")
    ap.add_argument("--config-iters", type=int, default=10)
    args = ap.parse_args()
    if args.summarize_traffic:
        print(json.dumps(summarize_traffic(*args.summarize_traffic, kernel=args.traffic_kernel)))
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads would be sharded across GPUs with no communication inside the path). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import block_sparse_attention_nabla_amd as nb
    import synth

    nb.load_library()
    dev = torch.device("cuda:0")
    w = synth.get_workload(args.workload)
    thr = w.thr_for(args.sparsity)
    log(f"workload {w.name}: B={w.B} H={w.H} S={w.S} D={w.D} n={w.n} thr={thr:.6f}")
    t0 = time.time()
    x = synth.make_inputs(w)
    log(f"inputs generated on the host in {time.time() - t0:.1f} s")
    q, k, v = (x[key].to(dev) for key in ("q", "k", "v"))
    B, H, S, D, n = w.B, w.H, w.S, w.D, w.n

    # Buffers and workspaces allocated once, outside the timed region.
    lists = {"kv_count": torch.empty((B, H, n), dtype=torch.int32, device=dev),
             "kv_idx": torch.empty((B, H, n, n), dtype=torch.int32, device=dev)}
    ws_mask = torch.empty(nb.nabla_workspace_size(nb.NABLA_OP_MASK, B, H, S, D), dtype=torch.uint8, device=dev)
    ws_fwd = torch.empty(nb.nabla_workspace_size(nb.NABLA_OP_FWD, B, H, S, D), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def mask_step():
        nb.nabla_build_mask(q, k, thr, w.sta_struct(), out=lists, workspace=ws_mask, stream=stream)

    # Scheduling hint: blocks per latent frame (the block order of section 3.1.1);
    # outputs are bitwise identical with or without it.
    fb = 0 if args.no_pairs else (w.Hs // w.P) * (w.Ws // w.P)

    def fwd_step(frame_blocks=None):
        nb.nabla_sparse_attn_fwd(q, k, v, lists["kv_count"], lists["kv_idx"], o=o, lse=lse,
                                 workspace=ws_fwd, stream=stream,
                                 frame_blocks=fb if frame_blocks is None else frame_blocks)

    for _ in range(args.warmup):
        mask_step()
        fwd_step()
    torch.cuda.synchronize()
    kept = int(lists["kv_count"].sum())
    sparsity = 1.0 - kept / (B * H * n * n)
    flops_per_kept = 4.0 * w.N * w.N * D
    step_flops = kept * flops_per_kept
    log(f"kept blocks {kept} -> sparsity {sparsity:.5f}; {step_flops / 1e12:.3f} TFLOP per step")

    # Timed region: exactly K steps; HIP events on the launch stream bracket
    # each stage so the forward kernel's own duration is known.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        mask_step()
        ev[i][1].record(stream)
        fwd_step()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    mask_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    fwd_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    fwd_each = sorted(e[1].elapsed_time(e[2]) for e in ev)
    mask_each = sorted(e[0].elapsed_time(e[1]) for e in ev)

    def pct(xs):
        def at(f):
            return xs[min(len(xs) - 1, int(round(f * (len(xs) - 1))))]
        return {"p10": round(at(0.1), 4), "p50": round(at(0.5), 4), "p90": round(at(0.9), 4)}
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    fwd_tflops = step_flops / (fwd_ms * 1e-3) / 1e12
    log(f"step {ms_per_step:.3f} ms (mask {mask_ms:.3f} ms, forward {fwd_ms:.3f} ms); "
        f"forward {fwd_tflops:.1f} TFLOP/s = {100 * fwd_tflops / PEAK_BF16_TFLOPS:.1f}% of peak")
    # The one-block-per-workgroup forward on the same lists, for reference.
    unpaired_ms = None
    if fb:
        e_u = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        fwd_step(0)
        e_u[0].record(stream)
        for _ in range(5):
            fwd_step(0)
        e_u[1].record(stream)
        torch.cuda.synchronize()
        unpaired_ms = e_u[0].elapsed_time(e_u[1]) / 5
        log(f"forward without the frame hint: {unpaired_ms:.3f} ms")

    # Cold caches: a 512 MB write before each call evicts L2 and the Infinity Cache.
    cold = None
    if args.cold_iters > 0:
        flush = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device=dev)
        ce = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.cold_iters)]
        for i in range(args.cold_iters):
            flush.fill_(i & 255)
            ce[i][0].record(stream)
            mask_step()
            ce[i][1].record(stream)
            flush.fill_((i + 1) & 255)
            fwd_step()
            ce[i][2].record(stream)
        torch.cuda.synchronize()
        cold = {"mask_ms": round(sum(e[0].elapsed_time(e[1]) for e in ce) / args.cold_iters, 4),
                "forward_ms": round(sum(e[1].elapsed_time(e[2]) for e in ce) / args.cold_iters, 4),
                "iters": args.cold_iters, "flush": "512 MB device write before each call"}
        del flush
        log(f"cold caches: {cold}")

    # Mask stage algorithmic bytes: read Q and K once, write counts and lists.
    mask_bytes = 2 * B * H * S * D * 2 + 4 * B * H * n + 4 * kept
    mask_gbps = mask_bytes / (mask_ms * 1e-3) / 1e9

    # Same kernel run dense: every block kept (thr >= 1).
    if args.no_dense:
        args.dense_iters = 0
    dense_ms = float("nan")
    if args.dense_iters > 0:
        dense_lists = {"kv_count": torch.empty_like(lists["kv_count"]), "kv_idx": torch.empty_like(lists["kv_idx"])}
        nb.nabla_build_mask(q, k, 1.0, out=dense_lists, workspace=ws_mask, stream=stream)
        nb.nabla_sparse_attn_fwd(q, k, v, dense_lists["kv_count"], dense_lists["kv_idx"], o=o, lse=lse,
                                 workspace=ws_fwd, stream=stream, frame_blocks=fb)
        torch.cuda.synchronize()
        dev_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.dense_iters)]
        for i in range(args.dense_iters):
            dev_ev[i][0].record(stream)
            nb.nabla_sparse_attn_fwd(q, k, v, dense_lists["kv_count"], dense_lists["kv_idx"], o=o, lse=lse,
                                     workspace=ws_fwd, stream=stream, frame_blocks=fb)
            dev_ev[i][1].record(stream)
        torch.cuda.synchronize()
        dense_ms = sum(e[0].elapsed_time(e[1]) for e in dev_ev) / args.dense_iters
        dense_flops = B * H * n * n * flops_per_kept
        speedup = dense_ms / fwd_ms
        log(f"dense forward {dense_ms:.2f} ms ({dense_flops / dense_ms / 1e9:.1f} TFLOP/s); "
            f"speedup {speedup:.2f}x at density {1 - sparsity:.4f} (linearity {speedup * (1 - sparsity):.3f})")
        del dense_lists
    sdpa_ms = dense_sdpa_ms(q, k, v, stream, args.dense_iters) if args.dense_iters > 0 else None

    # Mask fidelity: true block mass of dense attention (the dense run above left
    # the dense LSE in `lse`), and the recall of the 90% CDF lists.
    mass = None
    fidelity = None
    if args.dense_iters > 0 and not args.no_fidelity:
        mass = torch.empty((B, H, n, n), dtype=torch.float32, device=dev)
        nb.nabla_block_mass(q, k, lse, out=mass, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        nb.nabla_block_mass(q, k, lse, out=mass, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        mass_ms = e0.elapsed_time(e1)
        mass_flops = 2.0 * B * H * S * S * D
        fidelity = {
            "what": "dense attention mass inside the kept blocks vs the best blocks at the same per-row count",
            "block_mass_kernel_ms": round(mass_ms, 3),
            "block_mass_tflops": round(mass_flops / (mass_ms * 1e-3) / 1e12, 1),
            "cdf": recall_summary(nb, mass, lists),
        }
        log(f"fidelity: {fidelity}")

    if args.traffic_calibration:
        xa = torch.empty(CALIB_BYTES // 2, dtype=torch.bfloat16, device=dev).normal_()
        ya = torch.empty_like(xa)
        torch.mul(xa, 1.0, out=ya)  # plain copy kernel: reads and writes 1 GiB
        torch.cuda.synchronize()
        del xa, ya

    speedup = dense_ms / fwd_ms
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"{w.name}: B{B} H{H} D{D}, latent {w.T}x{w.Hs}x{w.Ws} = {S} tokens ({n} blocks), "
                         f"timed at {100 * sparsity:.0f}% block sparsity (other points under configs)"),
            "B": B, "H": H, "S": S, "D": D, "N": w.N,
            "thr": round(thr, 6), "block_sparsity": round(sparsity, 5),
            "step": "nabla_build_mask + nabla_sparse_attn_fwd (inputs resident in HBM)",
            "frame_blocks": fb,
        },
        "pct_of_bf16_peak_step": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "forward_tflops": round(fwd_tflops, 2),
        "forward_ms": round(fwd_ms, 4),
        "forward_unpaired_ms": round(unpaired_ms, 4) if unpaired_ms is not None else None,
        "forward_ms_percentiles": pct(fwd_each),
        "mask_ms_percentiles": pct(mask_each),
        "cold_caches": cold,
        "mask_ms": round(mask_ms, 4),
        "mask_gbps": round(mask_gbps, 1),
        "mask_pct_hbm_peak": round(100 * mask_gbps / PEAK_HBM_GBPS, 2),
        "dense_forward_ms": round(dense_ms, 3) if args.dense_iters > 0 else None,
        "speedup_vs_dense_forward": round(speedup, 3) if args.dense_iters > 0 else None,
        "speedup_vs_dense_with_mask": (round(dense_ms / (mask_ms + fwd_ms), 3)
                                       if args.dense_iters > 0 else None),
        # PyTorch's own dense attention on the same Q, K, V (flash backend forced): an
        # independent dense baseline beside this library's kernel run dense.
        "dense_torch_sdpa_ms": round(sdpa_ms, 3) if sdpa_ms else None,
        "speedup_vs_torch_sdpa_dense": round(sdpa_ms / fwd_ms, 3) if sdpa_ms else None,
        "linearity": round(speedup * (1 - sparsity), 3) if args.dense_iters > 0 else None,
        "load_balance_efficiency": (round((1 - sparsity) * dense_ms / fwd_ms, 3)
                                    if args.dense_iters > 0 else None),
        "roofline": {
            "kernel": FWD_KERNEL if fb else "attn_fwd_kernel",
            "bound": "mfma",
            "achieved": round(fwd_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(step_flops),
            "algorithmic_flop_per_launch": step_flops,
            "note": "forward call = pair-count kernel + per-head longest-first ordering kernel + the "
                    "attention kernel, events bracket all three; peak assumes 2.4 GHz while the GPU "
                    "runs at ~1.8-1.9 GHz under this load (counters: MFMA busy ~49% of SIMD cycles, "
                    "1/16 of it the MFMA weight sums); the kernel is limited by its per-block step "
                    "(~85 non-transcendental softmax VALU instructions per step that co-issue with "
                    "MFMA only in part) and by waits on union steps only one block of a pair keeps, "
                    "not by LDS (~21% busy) or by its traffic beyond L2 (see traffic; ~5.5 TB/s, "
                    "below the ~7 TB/s the one-block kernel sustains)",
        },
        "cpu_baseline": None,
        "context": {
            "note": "the pages' own end-to-end numbers, other hardware and metric: context, not targets",
            "inference": "2.72x faster than full attention for NABLA(0.4) at 92.5% sparsity (3.07 vs 8.35 min), "
                         "Wan 2.1 14B text-to-video at 720p, 4x H100 (Table 1)",
            "pretraining": "1.46x: 7.5 s vs 10.9 s per iteration, 2B DiT at 512x512 with 80% sparse NABLA, "
                           "hardware not stated (section 4.3)",
        },
    }
    if not args.no_configs:
        configs = {}
        if w.name == "wan14b_720p":
            # The other operating point of Table 1 on the same inputs, against the same dense run.
            other = 0.80 if abs(args.sparsity - 0.90) < 1e-6 else 0.90
            ws_pair = {nb.NABLA_OP_MASK: ws_mask, nb.NABLA_OP_FWD: ws_fwd}
            configs[f"wan14b_720p_{int(round(other * 100))}"] = sparse_point(
                nb, w, q, k, v, w.thr_for(other), stream, args.config_iters, fb,
                dense_ms=dense_ms if args.dense_iters > 0 else None, ws=ws_pair)
            log(f"720p at {other}: {configs[f'wan14b_720p_{int(round(other * 100))}']}")
            # The STA-union workload at the layer's own shape: the 90% CDF mask of the same
            # inputs OR the STA(11, 24, 24) window (per-row counts 24-535 blocks).
            sta720 = dict(T=w.T, Hs=w.Hs, Ws=w.Ws, P=w.P, win_t=11, win_h=24, win_w=24)
            configs["wan14b_720p_90_sta"] = sparse_point(
                nb, w, q, k, v, w.thr_for(0.90), stream, args.config_iters, fb,
                dense_ms=dense_ms if args.dense_iters > 0 else None, ws=ws_pair, sta=sta720)
            configs["wan14b_720p_90_sta"]["workload"] = (
                "wan14b_720p inputs, NABLA(thr of 90%) OR STA(11,24,24) (temporal +-5 frames, "
                "spatial 3x3 tiles)")
            log(f"720p STA union: {configs['wan14b_720p_90_sta']}")
        out_of_main = small_configs(nb, dev, stream, args)
        configs.update(out_of_main)
        result["configs"] = configs
    if not args.no_selectors:
        # Top-k at the CDF rule's mean kept count; STA at Table 1's (18, 24, 24) window.
        topk = max(1, round(kept / (B * H * n)))
        result["selectors"] = selector_bench(w, q, k, v, lists, ws_mask, ws_fwd, o, lse, stream, 5,
                                             topk, (18, 24, 24), mass, fb)
    if fidelity is not None:
        result["fidelity"] = fidelity
        del mass
    if not args.no_reorder:
        result["reorder"] = reorder_bench(w, dev, stream, args.reorder_iters)
    if not args.no_configs and w.name == "wan14b_720p":
        # Side figure: the same layer on the literal recipe (pooled-logit std 3),
        # whose rows are far more peaked (see the input-scale reading).
        ws3 = {nb.NABLA_OP_MASK: ws_mask, nb.NABLA_OP_FWD: ws_fwd}
        w3 = synth.get_workload("wan14b_720p_std3")
        x3 = synth.make_inputs(w3)
        q3, k3, v3 = (x3[key].to(dev) for key in ("q", "k", "v"))
        del x3
        std3 = {"workload": f"{w3.name}: {w3.description}"}
        for sp in (0.80, 0.90):
            std3[f"sparsity={sp:.2f}"] = sparse_point(
                nb, w3, q3, k3, v3, w3.thr_for(sp), stream, args.config_iters, fb,
                dense_ms=dense_ms if args.dense_iters > 0 else None, ws=ws3)
        result["configs"]["wan14b_720p_std3"] = std3
        log(f"std3 side figure: {std3}")
        del q3, k3, v3
    if not args.no_train:
        del o, lse, lists, ws_mask, ws_fwd, q, k, v
        torch.cuda.empty_cache()
        result["train_step"] = train_step(args, dev, stream)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        xc = {key: x[key] for key in ("q", "k", "v")}
        qh = xc["q"].reshape(-1, S, D)[:2].reshape(1, 2, S, D).to(dev)
        kh = xc["k"].reshape(-1, S, D)[:2].reshape(1, 2, S, D).to(dev)
        gm = nb.nabla_build_mask(qh, kh, thr, w.sta_struct(), dense=True)["dense_mask"]
        gpu_dense = gm.reshape(2, n, n).cpu().numpy()
        del qh, kh, gm
        result["cpu_baseline"] = cpu_baseline(w, xc, thr, gpu_dense_mask=gpu_dense)
        log(f"cpu baseline {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
