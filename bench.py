#!/usr/bin/env python3
"""Benchmark of the tiled exact attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dense_bf16] [--warm-seconds S]

One step is one call of the tiled attention forward (query-tile decomposition, Q load, K/V
tile stream, QK^T, scale and mask, online softmax, PV and the epilogue) over the dense bf16
workload B=4 H=32 N=1024 d=128, the configuration the throughput metric is quoted on. The
other workloads (fp16 dense, causal, sliding window + global keys, paged decode) are timed in
the same run and reported under "workloads", with chunked prefill against the paged cache,
multimodal attention (three calls merged by log-sum-exp, beside one prefix-LM call) and the
backward pass (dQ, dK, dV) of the dense, causal and block-sparse workloads. Prints one JSON
line.

Throughput counts 4*d FLOPs per visible (query, key) pair (QK^T and PV), with the exact pair
count of the mask (not whole tiles); decode counts algorithmic HBM bytes (K and V of every
visible key, the query, the output). Kernel durations come from HIP events recorded on the
stream the kernels run on. The oracle (fp64, CPU) is timed on a bounded sample of the same
workload as a reported baseline.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 MFMA
PAGES_F32_TFLOPS = 0.57     # pages' Ascend 910 fp32 time for the dense shape, as TFLOP/s
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PAGES_BF16_TFLOPS = 1.25    # pages' Ascend 910 bf16 time for this workload, as TFLOP/s
CSRC = "tiled_exact_attention_forward_amd/csrc/"
# Sources each measured kernel is compiled from (its traffic entry is valid for these only).
KERNEL_SOURCES = {
    "fwd": [CSRC + "fa_device.h", CSRC + "fa_fwd.hip"],
    "bwd": [CSRC + "fa_device.h", CSRC + "fa_bwd.hip"],
    "decode": [CSRC + "fa_launch.h", CSRC + "fa_decode.hip"],
    "merge": [CSRC + "fa_device.h", CSRC + "fa_merge.hip"],
}


# ----------------------------------------------------------------- accounting

def score_matrix_bytes(B, H, N, elem_bytes):
    """Bytes of a materialised N x N score matrix per (batch, head)."""
    return B * H * N * N * elem_bytes


def tile_bytes(rows, cols, elem_bytes, tiles=1):
    return rows * cols * elem_bytes * tiles


def visible_counts(Nq, Nkv, mode, W=0, G=0):
    """Visible keys of every query row (closed form, vectorised over rows)."""
    ip = np.arange(Nq, dtype=np.int64) + (Nkv - Nq)
    if mode == 0:
        return np.full(Nq, Nkv, dtype=np.int64)
    top = np.clip(np.minimum(ip, Nkv - 1) + 1, 0, None)
    if mode == 1:
        return top
    if mode == 3:
        return np.maximum(0, np.minimum(Nkv - 1, ip + W) - np.maximum(0, ip - W) + 1)
    if mode == 4:
        return np.minimum(Nkv, np.maximum(np.maximum(G, ip + 1), 0))
    start = np.maximum(0, ip - W + 1)
    in_win = np.maximum(0, top - start)
    glob = np.maximum(0, np.minimum(np.minimum(G, start), top))
    return in_win + glob


def block_sparse_pairs(layout, Nq, Nkv, block):
    """Visible (query, key) pairs of a block layout [H, nqb, nkb], summed over heads."""
    lay = np.asarray(layout, dtype=np.int64) != 0
    rows = np.minimum(block, Nq - block * np.arange(lay.shape[1]))
    keys = np.minimum(block, Nkv - block * np.arange(lay.shape[2]))
    return int((lay * rows[None, :, None] * keys[None, None, :]).sum())


def tile_elements(Nq, Nkv, mode, W=0, G=0, bm=128, bn=32, layout=None, block=128):
    """(query tile, key tile) pairs of bm x bn tiles holding at least one visible pair, and the
    elements of those tiles (partial tiles at the edges count their real rows and keys), for
    one (b, h); summed over heads for a block layout [H, nqb, nkb]. The tile-granular work
    behind the exact pair count."""
    i0 = np.arange(0, Nq, bm, dtype=np.int64)
    k0 = np.arange(0, Nkv, bn, dtype=np.int64)
    rows = np.minimum(bm, Nq - i0)
    cols = np.minimum(bn, Nkv - k0)
    if mode == 5:
        lay = np.asarray(layout, dtype=np.int64) != 0           # [H, nqb, nkb], bm == block
        vis = lay[:, :, np.minimum(k0 // block, lay.shape[2] - 1)]  # [H, nqt, nkt]
        return int(vis.sum()), int((vis * rows[None, :, None] * cols[None, None, :]).sum())
    p0 = (i0 + (Nkv - Nq))[:, None]                 # position of each tile's first row
    p1 = (i0 + rows - 1 + (Nkv - Nq))[:, None]      # and of its last row
    a, b = k0[None, :], (k0 + cols - 1)[None, :]     # first and last key of each key tile
    if mode == 0:
        vis = np.ones((len(i0), len(k0)), dtype=bool)
    elif mode == 1:
        vis = a <= p1
    elif mode == 2:
        vis = ((a < G) & (a <= p1)) | (np.maximum(p0, a) <= np.minimum(p1, b + W - 1))
    elif mode == 3:
        vis = (a <= p1 + W) & (b >= p0 - W)
    else:
        vis = (a <= p1) | (a < G)
    return int(vis.sum()), int((vis * rows[:, None] * cols[None, :]).sum())


def prefill_flops(w, layout=None):
    if w["mask"] == 5:
        pairs = block_sparse_pairs(layout, w["Nq"], w["Nkv"], w["block"]) * w["B"]
        return 4 * w["d"] * pairs, pairs
    pairs = int(visible_counts(w["Nq"], w["Nkv"], w["mask"], w["window"], w["n_global"]).sum())
    return 4 * w["d"] * pairs * w["B"] * w["H"], pairs * w["B"] * w["H"]


def prefill_bytes(w, elem):
    return elem * w["B"] * w["H"] * w["d"] * (2 * w["Nq"] + 2 * w["Nkv"]) + 4 * w["B"] * w["H"] * w["Nq"]


def decode_bytes(w, seq_lens, elem):
    keys = int(np.asarray(seq_lens, dtype=np.int64).sum())
    return 2 * keys * w["H"] * w["d"] * elem + 2 * w["S"] * w["H"] * w["d"] * elem + 4 * w["S"] * w["H"]


def kernel_source_hash(group=None):
    """Hash of the sources of one kernel group (all groups when None)."""
    h = hashlib.sha256()
    groups = [group] if group else sorted(KERNEL_SOURCES)
    for gname in groups:
        for p in KERNEL_SOURCES[gname]:
            with open(os.path.join(ROOT, p), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key):
    """HBM traffic per launch measured with rocprofv3 counters, if taken on the current
    sources of that kernel (each entry records the hash of its own sources)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get("kernels", {}).get(kernel_key)
    if e is None or e.get("source_hash") != kernel_source_hash(e.get("sources")):
        return None
    return e.get("bytes_per_launch")


def backward_traffic(workload):
    """Summed counter-measured HBM bytes of the two backward kernels, when measured."""
    parts = [load_traffic(f"bwd_{k}_bf16_d128_mask0_{workload}") for k in ("dq", "dkdv")]
    return None if any(p is None for p in parts) else sum(parts)


# ----------------------------------------------------------------- timing

# Untimed warm-up lasts at least this long (wall clock) besides the W warm-up steps: the
# GPU raises its clock over the first fraction of a second of load, and the first calls of
# a kernel in a process run slower; the timed steps measure the steady state.
MIN_WARM_S = 1.0


def time_calls(fn, steps, warmup, torch, min_warm_s=None):
    min_warm_s = MIN_WARM_S if min_warm_s is None else min_warm_s
    t_warm = time.perf_counter()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    while time.perf_counter() - t_warm < min_warm_s:
        for _ in range(max(1, warmup)):
            fn()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(stop) / steps, wall


def time_cold(fn, calls, torch, flush_bytes=1 << 30):
    """Per-call kernel time with L2 and MALL flushed before each call (a fill kernel writes a
    buffer larger than both, outside the timed region). Returns (median, min, p90) in ms."""
    scratch = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream()
    times = []
    for i in range(calls):
        scratch.fill_(i & 0xFF)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(stream)
        fn()
        stop.record(stream)
        stop.synchronize()
        times.append(start.elapsed_time(stop))
    del scratch
    t = np.sort(np.asarray(times))
    return float(np.median(t)), float(t[0]), float(t[min(len(t) - 1, int(0.9 * len(t)))])


def peak_fraction(r):
    """Rate against the datasheet MFMA peak of the workload's own dtype (fp32 inputs run
    fp32 MFMAs; the pages time the same dense shape in fp32 too)."""
    if r["w"]["dtype"] == "f32":
        return dict(frac_f32_peak=round(r["tflops"] / PEAK_F32_TFLOPS, 4),
                    pages_f32_tflops=PAGES_F32_TFLOPS,
                    note_f32="fp32 kernels are a plain path (fp32 products throughout)")
    return dict(frac_bf16_peak=round(r["tflops"] / PEAK_BF16_TFLOPS, 4))


def bench_prefill(name, steps, warmup, torch, fa, workloads, cold_calls=20):
    w, inp = workloads.gen_workload(name)
    dev = torch.device("cuda:0")
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    scale = workloads.default_scale(w["d"])

    if w["mask"] == 5:
        lay = inp["layout"].to(dev)

        def step():
            fa.fa_forward_block_sparse(q, k, v, lay, w["block"], scale, out=o, lse=lse)
    else:
        def step():
            fa.fa_forward(q, k, v, scale, w["mask"], w["window"], w["n_global"], out=o,
                          lse=lse)

    ms, wall = time_calls(step, steps, warmup, torch)
    cold = time_cold(step, cold_calls, torch) if cold_calls else (ms, ms, ms)
    flops, pairs = prefill_flops(w, inp.get("layout"))
    tiles, elems = tile_elements(w["Nq"], w["Nkv"], w["mask"], w["window"], w["n_global"],
                                 layout=inp.get("layout"))
    if w["mask"] != 5:
        tiles, elems = tiles * w["B"] * w["H"], elems * w["B"] * w["H"]
    else:
        tiles, elems = tiles * w["B"], elems * w["B"]
    elem = q.element_size()
    return dict(workload=name, w=w, ms=ms, wall_s=wall, flops=flops, pairs=pairs,
                tile_count=dict(tiles=tiles, elements=elems,
                                tflops=round(4 * w["d"] * elems / (ms * 1e-3) / 1e12, 2),
                                note="4*d FLOPs per element of every 128x32 (query x key) tile "
                                     "holding a visible pair; the headline counts visible "
                                     "pairs only"),
                tflops=flops / (ms * 1e-3) / 1e12, bytes=prefill_bytes(w, elem), inputs=inp,
                cold_ms=cold, cold_tflops=flops / (cold[0] * 1e-3) / 1e12)


def paged_prefill_pairs(w, seq_lens, q_lens):
    """Visible (query, key) pairs of a chunked prefill: chunk row i of sequence s is at
    absolute position i + L_s - n_s, with the workload's mask over L_s keys."""
    total = 0
    for L, n in zip(np.asarray(seq_lens, np.int64), np.asarray(q_lens, np.int64)):
        if n > 0:
            total += int(visible_counts(int(n), int(L), w["mask"], w["window"],
                                        w["n_global"]).sum())
    return total * w["H"]


def bench_prefill_paged(name, steps, warmup, torch, fa, workloads, cold_calls=20):
    w, inp = workloads.gen_workload(name)
    dev = torch.device("cuda:0")
    q, kp, vp, pt, sl, ql = (inp[x].to(dev) for x in ("q", "k_pages", "v_pages", "page_table",
                                                      "seq_lens", "q_lens"))
    o = torch.zeros_like(q)
    lse = torch.zeros(q.shape[:3], dtype=torch.float32, device=dev)
    scale = workloads.default_scale(w["d"])
    mask = (w["mask"], w["window"], w["n_global"])

    def step():
        fa.fa_prefill_paged(q, kp, vp, pt, sl, ql, scale, *mask, out=o, lse=lse)

    ms, wall = time_calls(step, steps, warmup, torch)
    cold = time_cold(step, cold_calls, torch) if cold_calls else (ms, ms, ms)
    pairs = paged_prefill_pairs(w, inp["seq_lens"], inp["q_lens"])
    flops = 4 * w["d"] * pairs
    return dict(workload=name, w=w, ms=ms, wall_s=wall, flops=flops, pairs=pairs,
                tflops=flops / (ms * 1e-3) / 1e12, cold_ms=cold,
                cold_tflops=flops / (cold[0] * 1e-3) / 1e12,
                seq_lens=[int(x) for x in inp["seq_lens"]],
                q_lens=[int(x) for x in inp["q_lens"]])


def multimodal_pairs(w):
    """Visible pairs of the multimodal pattern per (b, h): image x image, text x image, and
    text x text causally."""
    ni, nt = w["n_img"], w["n_txt"]
    return (ni * ni + nt * ni + nt * (nt + 1) // 2) * w["B"] * w["H"]


def bench_multimodal(name, steps, warmup, torch, fa, workloads, cold_calls=20):
    """The three-call split with its merge (fa_multimodal_forward) and, for comparison, one
    prefix-LM call over [image; text] (the unified mask)."""
    w, inp = workloads.gen_workload(name)
    dev = torch.device("cuda:0")
    qi, ki, vi, qt, kt, vt = (inp[x].to(dev) for x in ("q_img", "k_img", "v_img", "q_txt",
                                                       "k_txt", "v_txt"))
    scale = workloads.default_scale(w["d"])
    code = {"f32": fa.FA_F32, "f16": fa.FA_F16, "bf16": fa.FA_BF16}[w["dtype"]]
    ws = torch.empty((fa.fa_multimodal_workspace_bytes(w["B"], w["H"], w["n_txt"], w["d"],
                                                       code),), dtype=torch.uint8, device=dev)

    def split():
        fa.fa_multimodal_forward(qi, ki, vi, qt, kt, vt, scale, workspace=ws)

    q, k, v = (torch.cat([a, b], dim=2).contiguous() for a, b in ((qi, qt), (ki, kt), (vi, vt)))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    def unified():
        fa.fa_forward(q, k, v, scale, fa.FA_MASK_PREFIX_LM, 0, w["n_img"], out=o, lse=lse)

    def fused():
        fa.fa_multimodal_forward(qi, ki, vi, qt, kt, vt, scale,
                                 text_mode=fa.FA_MULTIMODAL_FUSED)

    ms, wall = time_calls(split, steps, warmup, torch)
    ms_f, _ = time_calls(fused, steps, warmup, torch)
    ms_u, _ = time_calls(unified, steps, warmup, torch)
    cold = time_cold(split, cold_calls, torch) if cold_calls else (ms, ms, ms)
    pairs = multimodal_pairs(w)
    flops = 4 * w["d"] * pairs
    return dict(workload=name, w=w, ms=ms, wall_s=wall, ms_unified=ms_u, ms_fused=ms_f,
                flops=flops, pairs=pairs, tflops=flops / (ms * 1e-3) / 1e12,
                tflops_fused=flops / (ms_f * 1e-3) / 1e12,
                tflops_unified=flops / (ms_u * 1e-3) / 1e12, cold_ms=cold)


def bench_backward(name, steps, warmup, torch, fa, workloads, cold_calls=20):
    """One fa_backward call (row statistics, dK/dV, dQ kernels) on a prefill workload, with
    O and LSE from one forward call made before the timed region."""
    w, inp = workloads.gen_workload(name)
    dev = torch.device("cuda:0")
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    do = workloads.gen_dout(tuple(q.shape), w["dtype"], w["seed"] + 500).to(dev)
    scale = workloads.default_scale(w["d"])
    mask = (w["mask"], w["window"], w["n_global"])
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty((fa.fa_backward_workspace_bytes(w["B"], w["H"], w["Nq"]),),
                     dtype=torch.uint8, device=dev)
    layout = None
    if w["mask"] == 5:  # block sparse: the forward's layout
        layout = inp["layout"]
        lay = layout.to(dev)
        o, lse = fa.fa_forward_block_sparse(q, k, v, lay, w["block"], scale)

        def step():
            fa.fa_backward_block_sparse(q, k, v, o, lse, do, lay, w["block"], scale, dq=dq,
                                        dk=dk, dv=dv, workspace=ws)
    else:
        o, lse = fa.fa_forward(q, k, v, scale, *mask)

        def step():
            fa.fa_backward(q, k, v, o, lse, do, scale, *mask, dq=dq, dk=dk, dv=dv,
                           workspace=ws)

    ms, wall = time_calls(step, steps, warmup, torch)
    cold = time_cold(step, cold_calls, torch) if cold_calls else (ms, ms, ms)
    fwd_flops, pairs = prefill_flops(w, layout)
    flops = fwd_flops // 4 * 10  # 10 d per visible pair: S, dP, dV, dK, dQ
    return dict(workload=name, w=w, ms=ms, wall_s=wall, flops=flops, pairs=pairs,
                tflops=flops / (ms * 1e-3) / 1e12, cold_ms=cold,
                cold_tflops=flops / (cold[0] * 1e-3) / 1e12)


def bench_decode(name, steps, warmup, torch, fa, workloads, cold_calls=20):
    w, inp = workloads.gen_workload(name)
    dev = torch.device("cuda:0")
    q, kp, vp, pt, sl = (inp[x].to(dev) for x in ("q", "k_pages", "v_pages", "page_table",
                                                  "seq_lens"))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    need = fa.fa_decode_paged_workspace_bytes(w["S"], w["H"], w["d"], pt.shape[1], w["page_size"])
    ws = torch.empty((need,), dtype=torch.uint8, device=dev)
    scale = workloads.default_scale(w["d"])

    def step():
        fa.fa_decode_paged(q, kp, vp, pt, sl, scale, out=o, lse=lse, workspace=ws)

    ms, wall = time_calls(step, steps, warmup, torch)
    cold = time_cold(step, cold_calls, torch) if cold_calls else (ms, ms, ms)
    nbytes = decode_bytes(w, inp["seq_lens"], q.element_size())
    return dict(workload=name, w=w, ms=ms, wall_s=wall, bytes=nbytes,
                gbs=nbytes / (ms * 1e-3) / 1e9, seq_lens=[int(x) for x in inp["seq_lens"]],
                cold_ms=cold, cold_gbs=nbytes / (cold[0] * 1e-3) / 1e9)


def cpu_baseline(res, budget_s):
    """fp64 oracle on a bounded, evenly spaced sample of the workload's query rows."""
    import oracle
    w, inp = res["w"], res["inputs"]
    total_rows = w["B"] * w["H"] * w["Nq"]
    scale = float(np.float32(1.0 / math.sqrt(w["d"])))
    counts = visible_counts(w["Nq"], w["Nkv"], w["mask"], w["window"], w["n_global"])

    def run(n):
        rows = np.unique(np.linspace(0, total_rows - 1, n).astype(np.int64))
        t0 = time.perf_counter()
        oracle.attention(inp["q"], inp["k"], inp["v"], scale, w["mask"], w["window"],
                         w["n_global"], rows=rows)
        dt = time.perf_counter() - t0
        flops = 4 * w["d"] * int(counts[rows % w["Nq"]].sum())
        return rows.size, dt, flops

    n, dt, _ = run(min(512, total_rows))
    target = int(min(total_rows, max(512, n * budget_s / max(dt, 1e-3))))
    n, dt, flops = run(target)
    reps = 1
    if n == total_rows:  # the whole workload fits the budget: repeat it to fill the budget
        reps = max(1, int(budget_s / max(dt, 1e-3)))
        t0 = time.perf_counter()
        for _ in range(reps):
            run(total_rows)
        dt = (time.perf_counter() - t0) / reps
    what = (f"the whole workload ({total_rows} query rows), run {reps} times" if n == total_rows
            else f"{n} of {total_rows} query rows (evenly spaced over batch, head, row)")
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=oracle.num_threads(),
                kind="oracle", seconds=dt * reps, cpu_model=host_cpu_model(),
                sample=f"{what} of {res['workload']}, fp64 C oracle with OpenMP")


def host_cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where it is not readable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    global MIN_WARM_S
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dense_bf16")
    ap.add_argument("--only-headline", action="store_true",
                    help="skip the other workloads and the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--warm-seconds", type=float, default=None,
                    help="untimed warm-up also lasts at least this many seconds per workload "
                         f"(default {MIN_WARM_S}; 0 with --profile-workload, for profilers)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run plain device copies of MIB MiB (for HBM counter scaling)")
    ap.add_argument("--profile-workload", default=None,
                    help="only run this workload for --steps calls (for profilers); no JSON")
    ap.add_argument("--profile-backward", action="store_true",
                    help="with --profile-workload: time the backward pass instead")
    args = ap.parse_args()
    if args.warm_seconds is None:
        args.warm_seconds = 0.0 if args.profile_workload else MIN_WARM_S
    MIN_WARM_S = args.warm_seconds
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU sharding)", file=sys.stderr)
        sys.exit(2)

    import torch
    import tiled_exact_attention_forward_amd as fa
    import workloads
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fa.load_library()

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copied {args.copy_calibration} MiB x {args.steps}", file=sys.stderr)
        return
    if args.profile_workload:
        kind = workloads.WORKLOADS[args.profile_workload]["kind"]
        fn = {"prefill": bench_prefill, "decode": bench_decode,
              "prefill_paged": bench_prefill_paged, "multimodal": bench_multimodal}[kind]
        if args.profile_backward:
            fn = bench_backward
        r = fn(args.profile_workload, args.steps, args.warmup, torch, fa, workloads, cold_calls=0)
        print(f"[bench] {args.profile_workload}: {r['ms'] * 1e3:.1f} us per call", file=sys.stderr)
        return

    head = bench_prefill(args.workload, args.steps, args.warmup, torch, fa, workloads)
    print(f"[bench] {args.workload}: {head['ms'] * 1e3:.1f} us/step, "
          f"{head['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    others = {}
    if not args.only_headline:
        for name in ("dense_f16", "dense_bf16", "causal_bf16", "window_bf16", "band_bf16",
                     "prefix_bf16", "blocksparse_bf16", "dense_f32"):
            if name == args.workload:
                continue
            r = bench_prefill(name, max(10, args.steps // 4), max(3, args.warmup // 4), torch, fa,
                              workloads)
            others[name] = dict(us=round(r["ms"] * 1e3, 2), tflops=round(r["tflops"], 2),
                                visible_pairs=r["pairs"],
                                cold_us_median_min_p90=[round(x * 1e3, 2) for x in r["cold_ms"]],
                                cold_tflops=round(r["cold_tflops"], 2),
                                tile_count=r["tile_count"])
            others[name].update(peak_fraction(r))
            print(f"[bench] {name}: {r['ms'] * 1e3:.1f} us, {r['tflops']:.1f} TFLOP/s",
                  file=sys.stderr, flush=True)
            del r
            torch.cuda.empty_cache()
        r = bench_prefill_paged("prefill_paged_bf16", max(10, args.steps // 4),
                                max(3, args.warmup // 4), torch, fa, workloads)
        others["prefill_paged_bf16"] = dict(
            us=round(r["ms"] * 1e3, 2), tflops=round(r["tflops"], 2),
            frac_bf16_peak=round(r["tflops"] / PEAK_BF16_TFLOPS, 4), visible_pairs=r["pairs"],
            cold_us_median_min_p90=[round(x * 1e3, 2) for x in r["cold_ms"]],
            cold_tflops=round(r["cold_tflops"], 2), seq_lens=r["seq_lens"], q_lens=r["q_lens"],
            note="chunked prefill against the paged cache, causal bottom-right")
        print(f"[bench] prefill_paged_bf16: {r['ms'] * 1e3:.1f} us, {r['tflops']:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
        del r
        r = bench_multimodal("multimodal_bf16", max(10, args.steps // 4),
                             max(3, args.warmup // 4), torch, fa, workloads)
        others["multimodal_bf16"] = dict(
            us=round(r["ms"] * 1e3, 2), tflops=round(r["tflops"], 2),
            frac_bf16_peak=round(r["tflops"] / PEAK_BF16_TFLOPS, 4), visible_pairs=r["pairs"],
            fused_us=round(r["ms_fused"] * 1e3, 2), fused_tflops=round(r["tflops_fused"], 2),
            unified_us=round(r["ms_unified"] * 1e3, 2),
            unified_tflops=round(r["tflops_unified"], 2),
            cold_us_median_min_p90=[round(x * 1e3, 2) for x in r["cold_ms"]],
            note="us/tflops: three calls (image full, text causal, text to image) + LSE merge; "
                 "fused_*: image call + one causal text call over [image; text] keys read from "
                 "both tensors; unified_*: one prefix-LM call over concatenated [image; text]")
        print(f"[bench] multimodal_bf16: split {r['ms'] * 1e3:.1f} us, fused "
              f"{r['ms_fused'] * 1e3:.1f} us, unified {r['ms_unified'] * 1e3:.1f} us",
              file=sys.stderr, flush=True)
        del r
        for name in ("dense_bf16", "causal_bf16", "blocksparse_bf16", "dense_f32"):
            r = bench_backward(name, max(10, args.steps // 4), max(3, args.warmup // 4), torch,
                               fa, workloads)
            others["backward_" + name] = dict(
                us=round(r["ms"] * 1e3, 2), tflops=round(r["tflops"], 2),
                visible_pairs=r["pairs"],
                cold_us_median_min_p90=[round(x * 1e3, 2) for x in r["cold_ms"]],
                cold_tflops=round(r["cold_tflops"], 2),
                traffic=backward_traffic(name),
                note="fa_backward (2 kernels); 10*d FLOPs per visible pair")
            others["backward_" + name].update(peak_fraction(r))
            print(f"[bench] backward {name}: {r['ms'] * 1e3:.1f} us, {r['tflops']:.1f} TFLOP/s",
                  file=sys.stderr, flush=True)
            del r
            torch.cuda.empty_cache()
        d = bench_decode("decode_f16", max(10, args.steps // 4), max(3, args.warmup // 4), torch,
                         fa, workloads)
        split_t = load_traffic("decode_split_f16_h16_s256_decode_f16")
        comb_t = load_traffic("decode_combine_f16_decode_f16")
        others["decode_f16"] = dict(us=round(d["ms"] * 1e3, 2), gbs=round(d["gbs"], 1),
                                    frac_hbm_peak=round(d["gbs"] / PEAK_HBM_GBS, 4),
                                    bytes=d["bytes"], seq_lens=d["seq_lens"],
                                    traffic=None if split_t is None or comb_t is None
                                    else split_t + comb_t,
                                    cold_us_median_min_p90=[round(x * 1e3, 2)
                                                            for x in d["cold_ms"]],
                                    cold_gbs=round(d["cold_gbs"], 1),
                                    note="split + combine kernels; us/gbs: back-to-back calls, "
                                         "cold_*: L2 and MALL flushed before each call")
        print(f"[bench] decode_f16: {d['ms'] * 1e3:.1f} us, {d['gbs']:.0f} GB/s",
              file=sys.stderr, flush=True)

    base = None
    if not args.no_cpu_baseline and not args.only_headline:
        base = cpu_baseline(head, args.cpu_seconds)
        print(f"[bench] cpu oracle: {base['value'] * 1e3:.2f} GFLOP/s on {base['cores']} threads",
              file=sys.stderr, flush=True)

    w = head["w"]
    achieved = head["flops"] / (head["ms"] * 1e-3) / 1e12
    f32 = w["dtype"] == "f32"
    peak = PEAK_F32_TFLOPS if f32 else PEAK_BF16_TFLOPS
    kernel_key = f"fwd16_{w['dtype']}_d{w['d']}_mask{w['mask']}_{args.workload}"
    mask_name = {0: "none", 1: "causal", 2: "window+global", 3: "band", 4: "prefix LM",
                 5: "block sparse"}[w["mask"]]
    line = {
        "metric": "attention fwd TFLOP/s & % bf16 MFMA peak; paged-decode HBM GB/s",
        "value": round(head["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_min_seconds": args.warm_seconds,
        "ms_per_step": round(head["ms"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(head["tflops"] / PAGES_BF16_TFLOPS, 2)
        if args.workload == "dense_bf16" else
        round(head["tflops"] / PAGES_F32_TFLOPS, 2) if args.workload == "dense_f32" else None,
        "dtype": w["dtype"],
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: B={w['B']} H={w['H']} Nq={w['Nq']} "
                               f"Nkv={w['Nkv']} d={w['d']} mask={w['mask']}",
                   "global_batch": w["B"], "seq_len": w["Nq"], "parallelism": "none"},
        "cold_cache": {"us_median_min_p90": [round(x * 1e3, 2) for x in head["cold_ms"]],
                       "tflops_median": round(head["cold_tflops"], 3),
                       "note": "L2 and MALL flushed (1 GiB fill) before each timed call"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": None if f32 else load_traffic(kernel_key),
                     "kernel": f"fwd32_kernel<d={w['d']}, mask {mask_name}>" if f32 else
                     f"fwd16_kernel<{w['dtype']}, d={w['d']}, mask {mask_name}>",
                     "flops_per_launch": head["flops"],
                     "algorithmic_bytes_per_launch": head["bytes"],
                     # the same kernel with L2 and MALL flushed before each call (median)
                     "achieved_cold": round(head["cold_tflops"], 3),
                     "frac_cold": round(head["cold_tflops"] / peak, 4)},
        "cpu_baseline": None if base is None else {
            k: (round(v, 6) if isinstance(v, float) else v) for k, v in base.items()},
        "workloads": others,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
