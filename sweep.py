"""Forward-kernel sweeps on one MI355X: tile shapes, and problem shapes for the per-round fit.

Tile sweep. The kernel's tile shape is fixed at compile time: W waves of 32 query rows per workgroup
(query tile BM = 32 W) and an S-slot LDS ring of 32-key K/V tiles (32 S keys of K and V on
chip per workgroup). The pages tune the query and key block sizes of their kernel by
measurement (ops-transformer article on gitcode.csdn.net, section 三.1, block-size table);
this script repeats that for gfx950: it builds the library once per (W, S) and times each
build on the same inputs.

    python sweep.py tiles --build    # hipcc, no GPU needed; builds go to _build/sweep/
    python sweep.py tiles --run      # on the GPU

Workloads: causal bf16 B4 H32 N4096 d128 (inputs 0.5 N(0,1)) and dense bf16 B4 H32 N1024
d128. Each build's output is compared with the default build's (the shapes change only the
order of the online-softmax updates). Timing: at least one second of calls before each
measurement (the clock rises under load), builds measured in rotated order over several
rounds, median reported.

Shape sweep. The forward launches one workgroup per 128-row query tile; with two workgroups
per CU a 256-CU MI355X runs 512 at once, so B * H * N / 128 tiles take B * H * N / 65536
rounds, and each workgroup walks N / 32 key tiles of 32 keys (steps). Timing dense bf16
attention (H 32, d 128, N(0,1) inputs) over shapes with 1 to 8 rounds and 32 to 128 steps and
fitting  time = a + b * rounds + c * rounds * steps  separates the cost of a round of
workgroups (Q loads and first tiles, output stores) from the cost of the steps themselves.
Every measurement follows at least a second of calls; the median of 5 batches of 20
back-to-back calls is reported.

    python sweep.py shapes           # on the GPU, the in-tree library
"""
import argparse
import concurrent.futures as cf
import ctypes
import os
import statistics
import subprocess
import sys
import time

import numpy as np

from tiled_exact_attention_forward_amd import build as lib_build

OUT = os.path.join(lib_build.BUILD, "sweep")
# (waves, ring slots): LDS per workgroup is 16 KB per slot; 160 KB per CU.
VARIANTS = [(2, 3), (4, 3), (4, 4), (4, 5), (8, 4), (8, 6), (8, 8)]


def lib_path(w, s):
    return os.path.join(OUT, f"w{w}s{s}.so")


def _build_one(ws):
    w, s = ws
    tmp = os.path.join(OUT, f"obj_w{w}s{s}")
    os.makedirs(tmp, exist_ok=True)
    objs = []
    for src in lib_build.SOURCES:
        obj = os.path.join(tmp, src + ".o")
        cmd = ["hipcc", *lib_build.FLAGS, *lib_build.EXTRA.get(src, []),
               f"-DFA_FWD_WAVES={w}", f"-DFA_FWD_STAGES={s}", "-c",
               os.path.join(lib_build.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src} (w{w} s{s}):\n{r.stderr}")
        objs.append(obj)
    subprocess.run(["hipcc", "-shared", "-fPIC", f"--offload-arch={lib_build.ARCH}", *objs,
                    "-o", lib_path(w, s)], check=True)
    return lib_path(w, s)


def build_all():
    os.makedirs(OUT, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=3) as ex:
        for p in ex.map(_build_one, VARIANTS):
            print("built", p, flush=True)


def _workloads(torch):
    g = torch.Generator(device="cpu").manual_seed(3)
    out = []
    for name, (B, H, N, mask, amp) in {"causal_bf16 B4 H32 N4096": (4, 32, 4096, 1, 0.5),
                                       "dense_bf16 B4 H32 N1024": (4, 32, 1024, 0, 1.0)}.items():
        q, k, v = [(amp * torch.randn((B, H, N, 128), generator=g)).to(torch.bfloat16).cuda()
                   for _ in range(3)]
        pairs = B * H * (N * (N + 1) // 2 if mask == 1 else N * N)
        out.append((name, B, H, N, mask, q, k, v, 4.0 * 128 * pairs))
    return out


def run_all(rounds):
    import torch
    libs = {}
    for w, s in VARIANTS:
        p = lib_path(w, s)
        if not os.path.exists(p):
            raise SystemExit(f"{p} missing: run with --build first")
        lib = ctypes.CDLL(p)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.fa_forward.argtypes = [vp] * 5 + [i] * 5 + [f] + [i] * 4 + [vp]
        lib.fa_forward.restype = ctypes.c_int
        libs[(w, s)] = lib
    ref_key = (4, 4)
    stream = torch.cuda.current_stream()
    results = {}
    for name, B, H, N, mask, q, k, v, flops in _workloads(torch):
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        args = [ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, o, lse)] + \
               [B, H, N, N, 128, 128 ** -0.5, mask, 0, 0, 2, ctypes.c_void_p(stream.cuda_stream)]
        times = {key: [] for key in libs}
        for r in range(rounds):
            keys = list(libs)
            keys = keys[r % len(keys):] + keys[:r % len(keys)]
            for key in keys:
                lib = libs[key]
                t0 = time.perf_counter()
                while time.perf_counter() - t0 < 1.0:
                    for _ in range(5):
                        if lib.fa_forward(*args) != 0:
                            raise RuntimeError(f"fa_forward failed for w{key[0]} s{key[1]}")
                    torch.cuda.synchronize()
                if r == 0:
                    results.setdefault(name, {})[key] = o.float().clone()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                n = 20 if N > 2048 else 100
                e0.record()
                for _ in range(n):
                    lib.fa_forward(*args)
                e1.record()
                torch.cuda.synchronize()
                times[key].append(e0.elapsed_time(e1) / n * 1e3)
        outs = results[name]
        print(f"\n{name}: median of {rounds} rounds")
        print("| waves | query tile | ring slots (keys on chip) | LDS per workgroup | workgroups per CU"
              " | us per call | TFLOP/s | max |dO| vs 4x4 |")
        print("|---|---|---|---|---|---|---|---|")
        for (w, s), ts in times.items():
            us = statistics.median(ts)
            lds_kb = 16 * s
            per_cu = min(8 // w, 160 // lds_kb)
            d = (outs[(w, s)] - outs[ref_key]).abs().max().item()
            print(f"| {w} | {32 * w} | {s} ({32 * s}) | {lds_kb} KB | {per_cu} | {us:.1f} | "
                  f"{flops / us / 1e6:.0f} | {d:.1e} |", flush=True)


SHAPES = [(2, 1024), (4, 1024), (8, 1024), (16, 1024), (2, 2048), (4, 2048), (2, 4096),
          (4, 4096)]


def run_shapes():
    import torch

    import tiled_exact_attention_forward_amd as fa
    fa.load_library()
    H, D, concurrent = 32, 128, 512
    g = torch.Generator(device="cpu").manual_seed(1)
    rows = []
    print("| B | N | rounds | steps per workgroup | us per call | TFLOP/s |")
    print("|---|---|---|---|---|---|")
    for B, N in SHAPES:
        q, k, v = [torch.randn((B, H, N, D), generator=g).to(torch.bfloat16).cuda()
                   for _ in range(3)]
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")

        def call():
            fa.fa_forward(q, k, v, D ** -0.5, fa.FA_MASK_NONE, out=o, lse=lse)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 1.0:
            for _ in range(5):
                call()
            torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                call()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 20 * 1e3)
        us = statistics.median(ts)
        rounds, steps = B * H * N / 128 / concurrent, N // 32
        rows.append((B, N, rounds, steps, us))
        print(f"| {B} | {N} | {rounds:g} | {steps} | {us:.1f} | "
              f"{4.0 * B * H * N * N * D / us / 1e6:.0f} |", flush=True)
    A = np.array([[1.0, r, r * s] for _, _, r, s, _ in rows])
    y = np.array([u for *_, u in rows])
    c, *_ = np.linalg.lstsq(A, y, rcond=None)
    step_flops = 4.0 * concurrent * 128 * 32 * D
    print(f"fit: {c[0]:.2f} us + {c[1]:.2f} us per round + {c[2]:.4f} us per step and round "
          f"(the steps at {step_flops / c[2] / 1e6:.0f} TFLOP/s)")
    for (B, N, r, s, u), p in zip(rows, A @ c):
        print(f"  B {B} N {N}: {u:.1f} us measured, {p:.1f} us fitted")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("what", choices=["tiles", "shapes"])
    ap.add_argument("--build", action="store_true", help="tiles: build every variant (no GPU)")
    ap.add_argument("--run", action="store_true", help="tiles: time every built variant")
    ap.add_argument("--rounds", type=int, default=5)
    a = ap.parse_args()
    if a.what == "shapes":
        run_shapes()
        return 0
    if not (a.build or a.run):
        ap.error("tiles: give --build and/or --run")
    if a.build:
        build_all()
    if a.run:
        run_all(a.rounds)
    return 0


if __name__ == "__main__":
    sys.exit(main())
