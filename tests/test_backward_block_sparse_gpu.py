"""Parity of the block-sparse backward (fa_backward_block_sparse through the C ABI) with the
fp64 oracle's gradients, on the GPU.

The HIP backward receives O and LSE from the HIP block-sparse forward; the oracle recomputes
everything in fp64 with the same layout. Small shapes compare every element over random
layouts with ragged query and key tails, query blocks that see no key block and key blocks
that no query block sees (their gradients must be exactly zero); the full-size block-sparse
workload compares every element, head by head. An all-ones layout must reproduce the
unmasked backward bit for bit (same kernels, same tile order), and an empty one must give
zero gradients. Tolerances are the backward's (gpu_util.check_grads).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import tiled_exact_attention_forward_amd as fa
import workloads
from gpu_util import check_grads, f64, to_dev
from pins import block_mask
from test_block_sparse_gpu import NMAX, longest_layout

pytestmark = pytest.mark.gpu


def run_bwd_bs(q, k, v, do, scale, layout):
    qd, kd, vd, gd = to_dev(q, k, v, do)
    lay = layout.to(qd.device)
    o, lse = fa.fa_forward_block_sparse(qd, kd, vd, lay, 128, scale)
    dq, dk, dv = fa.fa_backward_block_sparse(qd, kd, vd, o, lse, gd, lay, 128, scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def check_per_head(got, ref, dtype, label, inputs, scale, layout):
    """check_grads head by head: the structural zeros depend on each head's layout."""
    H = inputs[0].shape[1]
    Nq, Nkv = inputs[0].shape[2], inputs[1].shape[2]
    vis = block_mask(layout.numpy(), 128, Nq, Nkv)
    for h in range(H):
        sl = lambda t: t[:, h:h + 1]  # noqa: E731
        check_grads([sl(g) for g in got], [sl(np.asarray(r)) for r in ref], dtype,
                    f"{label} head {h}", tuple(sl(t) for t in inputs), scale, vis[h])


def layout_for(H, Nq, Nkv, density, seed):
    """A random layout with, where the shape allows, one query block that sees nothing and
    one key block that no query block sees."""
    g = torch.Generator("cpu").manual_seed(seed)
    nqb, nkb = -(-Nq // 128), -(-Nkv // 128)
    lay = (torch.rand((H, nqb, nkb), generator=g) < density).to(torch.uint8)
    if nqb > 1:
        lay[0, nqb - 1, :] = 0
    if nkb > 2:
        lay[H - 1, :, 1] = 0
    return lay


SHAPES = [(1, 1, 1, 1), (1, 2, 300, 300), (2, 1, 200, 457), (1, 2, 513, 129), (1, 1, 1, 333),
          (1, 3, 1000, 1000), (1, 2, 129, 640)]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("density", [0.3, 0.7])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_block_sparse_small(dtype, d, density, shape):
    B, H, Nq, Nkv = shape
    seed = zlib.crc32(repr(("bwdbs", dtype, d, density, shape)).encode()) % 100000
    q, k, v = workloads.gen_prefill(B, H, Nq, Nkv, d, dtype, seed)
    do = workloads.gen_dout((B, H, Nq, d), dtype, seed + 1)
    lay = layout_for(H, Nq, Nkv, density, seed + 2)
    scale = workloads.default_scale(d)
    got = run_bwd_bs(q, k, v, do, scale, lay)
    ref = oracle.attention_backward_block_sparse(q, k, v, do, scale, lay.numpy(), 128)
    check_per_head(got, ref, dtype, f"{dtype} d{d} p{density} {shape}", (q, k, v, do), scale,
                   lay)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_all_ones_layout_equals_unmasked_bitwise(dtype):
    q, k, v = workloads.gen_prefill(2, 2, 300, 420, 128, dtype, 31)
    do = workloads.gen_dout((2, 2, 300, 128), dtype, 32)
    lay = torch.ones((2, 3, 4), dtype=torch.uint8)
    got = run_bwd_bs(q, k, v, do, 0.0884, lay)
    qd, kd, vd, gd = to_dev(q, k, v, do)
    o, lse = fa.fa_forward(qd, kd, vd, 0.0884, 0)
    want = fa.fa_backward(qd, kd, vd, o, lse, gd, 0.0884, 0)
    torch.cuda.synchronize()
    for a, b in zip(got, want):
        assert torch.equal(a, b)


def test_empty_layout_gives_zero_gradients():
    q, k, v = workloads.gen_prefill(1, 2, 200, 300, 128, "bf16", 33)
    do = workloads.gen_dout((1, 2, 200, 128), "bf16", 34)
    got = run_bwd_bs(q, k, v, do, 0.0884, torch.zeros((2, 2, 3), dtype=torch.uint8))
    for g in got:
        assert torch.all(g == 0)


def test_backward_block_sparse_deterministic():
    q, k, v = workloads.gen_prefill(1, 4, 1000, 1000, 128, "bf16", 35)
    do = workloads.gen_dout((1, 4, 1000, 128), "bf16", 36)
    lay = layout_for(4, 1000, 1000, 0.5, 37)
    a = run_bwd_bs(q, k, v, do, 0.0884, lay)
    b = run_bwd_bs(q, k, v, do, 0.0884, lay)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# The fp64 backward oracle over the block-sparse workload's ~1.1e9 visible pairs takes about
# 15 s on 16 host threads.
@pytest.mark.timeout(900)
def test_backward_block_sparse_full_size():
    """Every gradient element of the block-sparse workload, head by head."""
    w, inp = workloads.gen_workload("blocksparse_bf16")
    B, H, Nq, d = inp["q"].shape
    do = workloads.gen_dout((B, H, Nq, d), w["dtype"], w["seed"] + 500)
    scale = workloads.default_scale(d)
    lay = inp["layout"]
    got = [torch.from_numpy(f64(g)) for g in run_bwd_bs(inp["q"], inp["k"], inp["v"], do,
                                                         scale, lay)]
    torch.cuda.empty_cache()
    ref = oracle.attention_backward_block_sparse(inp["q"], inp["k"], inp["v"], do, scale,
                                                 lay.numpy(), w["block"])
    check_per_head(got, ref, w["dtype"], "blocksparse_bf16", (inp["q"], inp["k"], inp["v"], do),
                   scale, lay)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("long_side", ["keys", "queries"])
def test_longest_block_lists(dtype, long_side):
    """2048 x 128 - 77 keys (the dQ kernel lists up to 2048 key blocks per query block) or
    query rows (the dK/dV kernel lists up to 2048 query blocks per key block) against 200 on
    the other side, every element; heads whose short-side block sees nothing must give zero
    gradients there."""
    Nq, Nkv = (200, NMAX) if long_side == "keys" else (NMAX, 200)
    q, k, v = workloads.gen_prefill(1, 2, Nq, Nkv, 64, dtype, 38)
    do = workloads.gen_dout((1, 2, Nq, 64), dtype, 39)
    lay = longest_layout(2, 2048, 40, transpose=long_side == "queries")
    got = run_bwd_bs(q, k, v, do, 0.125, lay)
    ref = oracle.attention_backward_block_sparse(q, k, v, do, 0.125, lay.numpy(), 128)
    ln = lay.numpy().astype(bool)
    for h in range(2):
        zero_rows = np.repeat(~ln[h].any(axis=1), 128)[:Nq]
        zero_keys = np.repeat(~ln[h].any(axis=0), 128)[:Nkv]
        sl = lambda t: t[:, h:h + 1]  # noqa: E731
        e = check_grads([sl(g) for g in got], [sl(np.asarray(r)) for r in ref], dtype,
                        f"longest lists {long_side} {dtype} head {h}",
                        tuple(sl(t) for t in (q, k, v, do)), 0.125, (zero_rows, zero_keys))
        print("longest lists", long_side, dtype, h, e)
