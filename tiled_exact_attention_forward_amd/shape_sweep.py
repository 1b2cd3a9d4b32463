"""Dense forward over rounds of workgroups and steps per workgroup, with a linear fit (MI355X).

    python -m tiled_exact_attention_forward_amd.shape_sweep     # on the GPU

The forward launches one workgroup per 128-row query tile; with two workgroups per CU a
256-CU MI355X runs 512 at once, so B * H * N / 128 tiles take B * H * N / 65536 rounds, and
each workgroup walks N / 32 key tiles of 32 keys (steps). Timing dense bf16 attention (H 32,
d 128, N(0,1) inputs) over shapes with 1 to 8 rounds and 32 to 128 steps and fitting

    time = a + b * rounds + c * rounds * steps

separates the cost of a round of workgroups (Q loads and first tiles, output stores) from the
cost of the steps themselves. Every measurement follows at least a second of calls (the clock
rises under load); the median of 5 batches of 20 back-to-back calls is reported.
"""
import statistics
import sys
import time

import numpy as np

SHAPES = [(2, 1024), (4, 1024), (8, 1024), (16, 1024), (2, 2048), (4, 2048), (2, 4096),
          (4, 4096)]
H, D, CONCURRENT = 32, 128, 512


def main():
    import torch

    import tiled_exact_attention_forward_amd as fa
    fa.load_library()
    g = torch.Generator(device="cpu").manual_seed(1)
    rows = []
    for B, N in SHAPES:
        q, k, v = [torch.randn((B, H, N, D), generator=g).to(torch.bfloat16).cuda()
                   for _ in range(3)]
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        call = lambda: fa.fa_forward(q, k, v, D ** -0.5, fa.FA_MASK_NONE, out=o, lse=lse)
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
        rounds, steps = B * H * N / 128 / CONCURRENT, N // 32
        rows.append((B, N, rounds, steps, us))
        print(f"| {B} | {N} | {rounds:g} | {steps} | {us:.1f} | "
              f"{4.0 * B * H * N * N * D / us / 1e6:.0f} |", flush=True)
    A = np.array([[1.0, r, r * s] for _, _, r, s, _ in rows])
    y = np.array([u for *_, u in rows])
    c, *_ = np.linalg.lstsq(A, y, rcond=None)
    step_flops = 4.0 * CONCURRENT * 128 * 32 * D
    print(f"fit: {c[0]:.2f} us + {c[1]:.2f} us per round + {c[2]:.4f} us per step and round "
          f"(the steps at {step_flops / c[2] / 1e6:.0f} TFLOP/s)")
    for (B, N, r, s, u), p in zip(rows, A @ c):
        print(f"  B {B} N {N}: {u:.1f} us measured, {p:.1f} us fitted")
    return 0


if __name__ == "__main__":
    sys.exit(main())
