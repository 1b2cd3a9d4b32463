"""Block-sparse forward (fa_forward_block_sparse) against the fp64 oracle on the GPU.

Small shapes compare every element over random layouts (including query blocks with no
visible key block, and ragged query and key tails); the full-size workload compares every
element. An all-ones layout must reproduce the unmasked forward pass bit for bit (same
kernel, same tile order).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import tiled_exact_attention_forward_amd as fa
import workloads
from gpu_util import check, f64, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def run_bs(q, k, v, layout, scale):
    qd, kd, vd = to_dev(q, k, v)
    o, lse = fa.fa_forward_block_sparse(qd, kd, vd, layout.to(qd.device), 128, scale)
    torch.cuda.synchronize()
    return o, lse


SHAPES = [(1, 1, 1, 1), (1, 2, 128, 128), (2, 3, 200, 300), (1, 2, 300, 200), (1, 1, 513, 257),
          (1, 2, 64, 1000), (1, 1, 1000, 64)]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("density", [0.0, 0.3, 1.0])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_small_shapes(dtype, d, density, shape):
    B, H, Nq, Nkv = shape
    seed = zlib.crc32(repr((dtype, d, density, shape)).encode()) % 100000
    q, k, v = workloads.gen_prefill(B, H, Nq, Nkv, d, dtype, seed)
    g = torch.Generator("cpu").manual_seed(seed + 1)
    nqb, nkb = -(-Nq // 128), -(-Nkv // 128)
    lay = (torch.rand((H, nqb, nkb), generator=g) < density).to(torch.uint8)
    scale = workloads.default_scale(d)
    o, lse = run_bs(q, k, v, lay, scale)
    ro, rl = oracle.attention_block_sparse(q, k, v, scale, lay.numpy(), 128)
    check(o, lse, ro, rl, dtype, f"block sparse {dtype} d{d} p{density} {shape}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_all_ones_layout_equals_unmasked_bitwise(dtype):
    q, k, v = workloads.gen_prefill(2, 2, 300, 420, 128, dtype, 21)
    lay = torch.ones((2, 3, 4), dtype=torch.uint8)
    o, lse = run_bs(q, k, v, lay, 0.0884)
    qd, kd, vd = to_dev(q, k, v)
    o0, l0 = fa.fa_forward(qd, kd, vd, 0.0884, 0)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(lse, l0)


def test_empty_layout_rows_give_zero_and_minus_inf():
    q, k, v = workloads.gen_prefill(1, 2, 256, 256, 128, "bf16", 22)
    lay = torch.zeros((2, 2, 2), dtype=torch.uint8)
    lay[0, 1, 0] = 1
    o, lse = run_bs(q, k, v, lay, 0.0884)
    of, lf = f64(o), f64(lse)
    assert np.all(of[0, 0, :128] == 0) and np.all(np.isneginf(lf[0, 0, :128]))
    assert np.all(of[0, 1] == 0) and np.all(np.isneginf(lf[0, 1]))
    assert np.all(np.isfinite(lf[0, 0, 128:]))
    ro, rl = oracle.attention_block_sparse(q, k, v, 0.0884, lay.numpy(), 128)
    check(o, lse, ro, rl, "bf16", "empty rows")


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_never_reads_past_the_keys(dtype):
    dev = require_gpu()
    B, H, Nq, Nkv, d = 1, 2, 150, 200, 128
    q, k, v = workloads.gen_prefill(B, H, Nq, Nkv, d, dtype, 23)
    n = k.numel()
    pad = 64 * 128 * 4
    ks = torch.full((n + pad,), float("nan"), dtype=k.dtype, device=dev)
    vs = torch.full((n + pad,), float("nan"), dtype=k.dtype, device=dev)
    ks[:n] = k.reshape(-1).to(dev)
    vs[:n] = v.reshape(-1).to(dev)
    lay = torch.ones((H, 2, 2), dtype=torch.uint8)
    lay[1, 0, 1] = 0
    o, lse = fa.fa_forward_block_sparse(q.to(dev), ks[:n].view(k.shape), vs[:n].view(v.shape),
                                        lay.to(dev), 128, 0.0884)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_block_sparse(q, k, v, 0.0884, lay.numpy(), 128)
    check(o, lse, ro, rl, dtype, "nan canary block sparse")


@pytest.mark.timeout(600)
def test_full_size_every_element():
    w, inp = workloads.gen_workload("blocksparse_bf16")
    scale = workloads.default_scale(w["d"])
    o, lse = run_bs(inp["q"], inp["k"], inp["v"], inp["layout"], scale)
    ro, rl = oracle.attention_block_sparse(inp["q"], inp["k"], inp["v"], scale,
                                           inp["layout"].numpy(), w["block"])
    e = check(o, lse, ro, rl, w["dtype"], "blocksparse_bf16")
    print("blocksparse_bf16", e)


# The longest sequence the block-sparse entry points take is 2048 blocks of 128 positions;
# 77 short of it, the last key block is partial.
NMAX = 2048 * 128 - 77


def longest_layout(nqb, nkb, seed, transpose=False):
    """Layout [2, nqb, nkb] for one short side (2 blocks) against 2048 blocks on the other.
    Head 0: one short-side block sees every long-side block (a full 2048-entry block list on
    chip), the other a 3 % spread that includes the first and the last (partial) block.
    Head 1: one short-side block sees nothing, the other only the last block."""
    g = torch.Generator("cpu").manual_seed(seed)
    n = max(nqb, nkb)
    lay = torch.zeros((2, 2, n), dtype=torch.uint8)
    lay[0, 0] = (torch.rand(n, generator=g) < 0.03).to(torch.uint8)
    lay[0, 0, 0] = lay[0, 0, n - 1] = 1
    lay[0, 1] = 1
    lay[1, 1, n - 1] = 1
    return lay.transpose(1, 2).contiguous() if transpose else lay


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_longest_key_block_list(dtype):
    """Nkv = 2048 x 128 - 77, every element: the query tiles' key-block lists fill every
    compaction chunk, and rows that see no block give O = 0, LSE = -inf."""
    q, k, v = workloads.gen_prefill(1, 2, 200, NMAX, 64, dtype, 24)
    lay = longest_layout(2, 2048, 25)
    o, lse = run_bs(q, k, v, lay, 0.125)
    ro, rl = oracle.attention_block_sparse(q, k, v, 0.125, lay.numpy(), 128)
    e = check(o, lse, ro, rl, dtype, f"longest key-block list {dtype}")
    assert np.all(f64(o)[0, 1, :128] == 0) and np.all(np.isneginf(f64(lse)[0, 1, :128]))
    print("longest key-block list", dtype, e)
