"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Small shapes compare every element and span several tiles plus ragged tails; the full-size
workloads run in the same launch configuration the benchmark times and compare every
element as well. Tolerances are stated in gpu_util.
"""
import zlib

import pytest
import torch

import oracle
import tiled_exact_attention_forward_amd as fa
import workloads
from gpu_util import check, to_dev

pytestmark = pytest.mark.gpu


def run_fwd(q, k, v, scale, mask=0, W=0, G=0):
    qd, kd, vd = to_dev(q, k, v)
    o, lse = fa.fa_forward(qd, kd, vd, scale, mask, W, G)
    torch.cuda.synchronize()
    return o, lse


def run_decode(inp, scale):
    q, kp, vp, pt, sl = to_dev(inp["q"], inp["k_pages"], inp["v_pages"], inp["page_table"],
                               inp["seq_lens"])
    o, lse = fa.fa_decode_paged(q, kp, vp, pt, sl, scale)
    torch.cuda.synchronize()
    return o, lse


MASKS = [(0, 0, 0), (1, 0, 0), (2, 40, 5), (2, 1, 0), (2, 100, 70), (2, 64, 64), (2, 200, 130),
         (2, 65, 63), (3, 0, 0), (3, 33, 0), (3, 200, 0), (3, 1000, 0), (4, 0, 0), (4, 0, 63),
         (4, 0, 130), (4, 0, 1000)]
SHAPES = [(1, 1, 1, 1), (1, 2, 17, 17), (2, 3, 100, 100), (1, 2, 129, 129), (1, 1, 300, 300),
          (1, 2, 64, 200), (1, 2, 200, 64), (1, 1, 1, 333), (1, 2, 257, 513)]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", MASKS, ids=lambda m: f"m{m[0]}w{m[1]}g{m[2]}")
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_small_shapes(dtype, d, mask, shape):
    B, H, Nq, Nkv = shape
    seed = zlib.crc32(repr((dtype, d, mask, shape)).encode()) % 100000
    q, k, v = workloads.gen_prefill(B, H, Nq, Nkv, d, dtype, seed)
    scale = workloads.default_scale(d)
    o, lse = run_fwd(q, k, v, scale, *mask)
    ro, rl = oracle.attention(q, k, v, scale, *mask)
    check(o, lse, ro, rl, dtype, f"{dtype} d{d} mask{mask} {shape}")


# More 128-row query tiles than two workgroups per CU hold at once (512 on a 256-CU device),
# so the tiles run in several rounds of workgroups, compared on every element: ragged Nq and
# Nkv, key-tile counts of every residue mod the ring depth of 4, a single masked key tile,
# and a negative scale.
MANY_TILE_SHAPES = [
    (1, 64, 1100, 333, 128, "bf16", 1),   # 576 query tiles, 11 key tiles, tail masked
    (3, 40, 700, 70, 64, "f16", 1),       # 720 query tiles, 3 key tiles
    (1, 130, 520, 31, 128, "f16", 1),     # 650 query tiles, one masked key tile
    (4, 32, 1536, 64, 64, "bf16", 1),     # 1536 query tiles (three rounds), 2 key tiles
    (1, 32, 2125, 1000, 128, "bf16", 1),  # 544 query tiles, 32 key tiles, tail masked
    (2, 40, 900, 100, 128, "bf16", -1),   # 640 query tiles, 4 key tiles, negative scale
]


@pytest.mark.parametrize("shape", MANY_TILE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_dense_many_query_tiles(shape):
    B, H, Nq, Nkv, d, dtype, sign = shape
    seed = zlib.crc32(repr(("many", shape)).encode()) % 100000
    q, k, v = workloads.gen_prefill(B, H, Nq, Nkv, d, dtype, seed)
    scale = sign * workloads.default_scale(d)
    o, lse = run_fwd(q, k, v, scale, 0)
    ro, rl = oracle.attention(q, k, v, scale, 0)
    check(o, lse, ro, rl, dtype, f"{shape}")


def test_tiny_f32_workload():
    w, inp = workloads.gen_workload("tiny_f32")
    scale = workloads.default_scale(w["d"])
    o, lse = run_fwd(inp["q"], inp["k"], inp["v"], scale, w["mask"])
    ro, rl = oracle.attention(inp["q"], inp["k"], inp["v"], scale, w["mask"])
    e = check(o, lse, ro, rl, "f32", "tiny_f32")
    print("tiny_f32", e)


@pytest.mark.parametrize("name", ["dense_f16", "dense_bf16"])
def test_dense_full_size_every_element(name):
    w, inp = workloads.gen_workload(name)
    scale = workloads.default_scale(w["d"])
    o, lse = run_fwd(inp["q"], inp["k"], inp["v"], scale, w["mask"])
    ro, rl = oracle.attention(inp["q"], inp["k"], inp["v"], scale, w["mask"])
    e = check(o, lse, ro, rl, w["dtype"], name)
    print(name, e)


# Every output element of the long masked workloads, in the launch configuration the
# benchmark times. The oracle covers them in about a minute on 16 host threads (causal 550
# GFLOP, window 1.1 TFLOP, band 2.1 TFLOP, prefix 0.6 TFLOP at 4 d FLOPs per visible pair).
@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["causal_bf16", "window_bf16", "band_bf16", "prefix_bf16"])
def test_masked_full_size_every_element(name):
    w, inp = workloads.gen_workload(name)
    scale = workloads.default_scale(w["d"])
    o, lse = run_fwd(inp["q"], inp["k"], inp["v"], scale, w["mask"], w["window"], w["n_global"])
    ro, rl = oracle.attention(inp["q"], inp["k"], inp["v"], scale, w["mask"], w["window"],
                              w["n_global"])
    e = check(o, lse, ro, rl, w["dtype"], name)
    print(name, e)


def test_decode_full_size_every_element():
    w, inp = workloads.gen_workload("decode_f16")
    scale = workloads.default_scale(w["d"])
    o, lse = run_decode(inp, scale)
    ro, rl = oracle.decode_paged(inp["q"], inp["k_pages"], inp["v_pages"], inp["page_table"],
                                 inp["seq_lens"], scale)
    e = check(o, lse, ro, rl, "f16", "decode_f16")
    print("decode_f16", e)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("lens,max_len", [([1, 2, 63, 64, 65, 255, 256, 257], 8192),
                                          ([8192, 4096, 7000, 1], 8192),
                                          ([16000, 300, 16384], 16384)])
def test_decode_ragged_lengths(dtype, lens, max_len):
    w, inp = workloads.gen_workload("decode_f16", dtype=dtype, lens=lens, S=len(lens), H=16,
                                    max_len=max_len)
    scale = workloads.default_scale(w["d"])
    o, lse = run_decode(inp, scale)
    ro, rl = oracle.decode_paged(inp["q"], inp["k_pages"], inp["v_pages"], inp["page_table"],
                                 inp["seq_lens"], scale)
    check(o, lse, ro, rl, dtype, f"decode {dtype} {lens}")


@pytest.mark.timeout(600)
def test_decode_longest_sequence():
    """The longest sequence decode takes: 65535 pages of 256 tokens, so 65535 splits in the
    split pass's launch grid and 65535 partial results per head in the combine. The table
    maps its pages at random onto the 97 full pages of a cache drawn by the usual recipe
    (pages shared between positions, as a prefix cache shares them), so the pool stays
    small; a short sequence shares the launch."""
    maxp = 65535
    _, inp = workloads.gen_workload("decode_f16", dtype="f16", lens=[97 * 256, 300], S=2, H=8,
                                    max_len=97 * 256)
    g = torch.Generator("cpu").manual_seed(72)
    full = inp["page_table"][0, :97]
    pt = torch.full((2, maxp), -1, dtype=torch.int32)
    pt[0] = full[torch.randint(0, 97, (maxp,), generator=g)]
    pt[1, :2] = inp["page_table"][1, :2]
    inp = dict(inp, page_table=pt, seq_lens=torch.tensor([maxp * 256, 300], dtype=torch.int32))
    scale = workloads.default_scale(128)
    o, lse = run_decode(inp, scale)
    ro, rl = oracle.decode_paged(inp["q"], inp["k_pages"], inp["v_pages"], pt, inp["seq_lens"],
                                 scale)
    e = check(o, lse, ro, rl, "f16", "decode, longest sequence")
    print("decode longest sequence", e)
