"""Parity of the backward pass (fa_backward through the C ABI) with the fp64 oracle's
gradients, on the GPU.

The HIP backward receives O and LSE from the HIP forward (the chain a caller runs); the
oracle recomputes everything from q, k, v and dO in fp64. Small shapes compare every element
over several tiles and ragged tails for every mask; the full-size workloads (dense, causal,
prefix LM, window and band at N = 32768) run in the benchmark's launch configuration and
compare every gradient element, head by head.

Tolerance (gradients are sums of many products whose operands P and dS are rounded to the
16-bit type, u = 2^-8 for bf16 and 2^-11 for fp16, and D_i uses the forward's rounded O; the
float32 backward rounds nothing to 16 bits and takes u = 2^-16, derived in gpu_util):
  * max |g_gpu - g_ref| <= 8u * max |g_ref| + F over each gradient tensor, and
    ||g_gpu - g_ref||_2 <= 4u * ||g_ref||_2 (three roundings of relative size <= u/2 each);
  * F is the float32 accumulation floor of dS = P (dP - D): both dP_ij and D_i are d-term
    dot products of size <= max|dO| max|V| (O is a convex combination of V rows), so with
    gamma_d = d 2^-24 (Higham's bound) and a 16x margin for the order of the sums,
    F = |scale| * 2 d 2^-20 * max|dO| max|V| max(max|Q|, max|K|) for dQ and dK, 0 for dV.
    It matters only where dQ and dK vanish analytically (every row sees one key, so
    dP = D); there the rel-L2 gate is skipped;
  * structural zeros (rows without a visible key in dQ, keys no row sees in dK and dV) are
    exactly zero.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import tiled_exact_attention_forward_amd as fa
import workloads
from gpu_util import U_GRAD as U, check_grads, f64, to_dev
from pins import band_mask

pytestmark = pytest.mark.gpu

def run_bwd(q, k, v, do, scale, mask=0, W=0, G=0):
    qd, kd, vd, gd = to_dev(q, k, v, do)
    o, lse = fa.fa_forward(qd, kd, vd, scale, mask, W, G)
    dq, dk, dv = fa.fa_backward(qd, kd, vd, o, lse, gd, scale, mask, W, G)
    torch.cuda.synchronize()
    return dq, dk, dv


MASKS = [(0, 0, 0), (1, 0, 0), (2, 40, 5), (2, 1, 0), (2, 100, 70), (2, 65, 63), (3, 0, 0),
         (3, 33, 0), (3, 200, 0), (4, 0, 0), (4, 0, 63), (4, 0, 130), (4, 0, 1000)]
SHAPES = [(1, 1, 1, 1), (1, 2, 17, 17), (2, 3, 100, 100), (1, 2, 129, 129), (1, 1, 300, 300),
          (1, 2, 64, 200), (1, 2, 200, 64), (1, 1, 1, 333), (1, 2, 257, 513)]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", MASKS, ids=lambda m: f"m{m[0]}w{m[1]}g{m[2]}")
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_small(dtype, d, mask, shape):
    B, H, Nq, Nkv = shape
    seed = zlib.crc32(repr(("bwd", dtype, d, mask, shape)).encode()) % 100000
    q, k, v = workloads.gen_prefill(B, H, Nq, Nkv, d, dtype, seed)
    do = workloads.gen_dout((B, H, Nq, d), dtype, seed + 1)
    scale = workloads.default_scale(d)
    got = run_bwd(q, k, v, do, scale, *mask)
    ref = oracle.attention_backward(q, k, v, do, scale, *mask)
    check_grads(got, ref, dtype, f"{dtype} d{d} mask{mask} {shape}", (q, k, v, do), scale,
                band_mask(Nq, Nkv, *mask))


def test_backward_negative_scale_and_large_inputs():
    """A negative scale flips which keys dominate; inputs x8 make P close to one-hot."""
    q, k, v = workloads.gen_prefill(1, 2, 200, 300, 128, "bf16", 91, input_scale=8.0)
    do = workloads.gen_dout((1, 2, 200, 128), "bf16", 92)
    for scale in (-workloads.default_scale(128), workloads.default_scale(128)):
        for mask in ((0, 0, 0), (1, 0, 0), (3, 20, 0)):
            got = run_bwd(q, k, v, do, scale, *mask)
            ref = oracle.attention_backward(q, k, v, do, scale, *mask)
            check_grads(got, ref, "bf16", f"scale {scale} mask {mask}", (q, k, v, do), scale,
                        band_mask(200, 300, *mask))


def test_backward_zero_and_subnormal_scale():
    """scale 0, or a scale whose product with log2 e is subnormal (either sign), makes P uniform
    over each row's visible keys; hidden scores must still give P = 0."""
    q, k, v = workloads.gen_prefill(1, 2, 100, 150, 128, "bf16", 93)
    do = workloads.gen_dout((1, 2, 100, 128), "bf16", 94)
    u = U["bf16"]
    for scale in (0.0, 1e-39, -1e-39):
        for mask in ((0, 0, 0), (1, 0, 0), (2, 20, 3), (3, 10, 0)):
            got = run_bwd(q, k, v, do, scale, *mask)
            ref = oracle.attention_backward(q, k, v, do, scale, *mask)
            label = f"scale {scale} mask {mask}"
            if scale == 0.0:
                check_grads(got, ref, "bf16", label, (q, k, v, do), scale,
                            band_mask(100, 150, *mask))
                continue
            # dQ and dK are ~1e-39 (scale times O(1)), subnormal in the output type: only
            # finite and tiny; dV carries P and is compared as usual
            for g in got[:2]:
                g = f64(g)
                assert np.isfinite(g).all() and np.abs(g).max() < 1e-30, label
            g, r = f64(got[2]), np.asarray(ref[2], np.float64).reshape(got[2].shape)
            assert np.abs(g - r).max() <= 8 * u * np.abs(r).max(), label
            assert np.linalg.norm(g - r) <= 4 * u * np.linalg.norm(r), label


def test_backward_deterministic():
    q, k, v = workloads.gen_prefill(2, 4, 640, 640, 128, "bf16", 93)
    do = workloads.gen_dout((2, 4, 640, 128), "bf16", 94)
    scale = workloads.default_scale(128)
    a = run_bwd(q, k, v, do, scale, 1)
    b = run_bwd(q, k, v, do, scale, 1)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def full_size_every_head(name):
    """Every gradient element of a full-size workload, checked head by head (the tolerance of
    check_grads scales with each head's own largest gradient)."""
    w, inp = workloads.gen_workload(name)
    B, H, Nq, d = inp["q"].shape
    do = workloads.gen_dout((B, H, Nq, d), w["dtype"], w["seed"] + 500)
    scale = workloads.default_scale(d)
    mask = (w["mask"], w["window"], w["n_global"])
    got = [f64(g) for g in run_bwd(inp["q"], inp["k"], inp["v"], do, scale, *mask)]
    torch.cuda.empty_cache()
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], do, scale, *mask)
    vis = band_mask(Nq, inp["k"].shape[2], *mask)
    vis = (~vis.any(dim=1).numpy(), ~vis.any(dim=0).numpy())
    for b in range(B):
        for h in range(H):
            sl = lambda t: t[b:b + 1, h:h + 1]  # noqa: E731
            ins = tuple(sl(t) for t in (inp["q"], inp["k"], inp["v"], do))
            check_grads([torch.from_numpy(sl(g)) for g in got], [sl(r) for r in ref],
                        w["dtype"], f"{name} head ({b},{h})", ins, scale, vis)


# The fp64 backward oracle takes 1280 FLOPs per visible pair (10 d): about 2 s for the dense
# workload, 20 s causal, 20 s prefix, 35 s window and 70 s band on 16 host threads.
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["dense_bf16", "causal_bf16", "prefix_bf16", "window_bf16",
                                  "band_bf16"])
def test_backward_full_size(name):
    full_size_every_head(name)
