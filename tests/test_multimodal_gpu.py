"""Parity of the log-sum-exp merge (fa_merge_lse) and of multimodal attention
(fa_multimodal_forward: image full, text causal, text-to-image, merged) with the fp64 oracle,
through the C ABI, on the GPU.

The merge is compared with the oracle's merge on the same float32 statistics and
dtype-valued partial outputs, with empty sides (lse = -inf); in place must equal out of
place bitwise. Multimodal attention is compared with the oracle's plain definition (one
attention over [image; text] with the multimodal visibility), and with the single
prefix-LM call of the forward kernel over [image; text] (the article states the split is
numerically the same as one call). Tolerances: the forward's (gpu_util) for O and LSE; the
merge rounds once to dtype (|err| <= 2^-8 |o| for bf16, 2^-11 for fp16, 2^-24 for fp32, plus
float32 arithmetic) and its LSE is float32 (|err| <= 4 2^-24 max(1, |lse|)).
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import tiled_exact_attention_forward_amd as fa
import workloads
from gpu_util import check, f64, to_dev

pytestmark = pytest.mark.gpu

REL = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -22}


def merge_inputs(rows, d, dtype, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    oa = torch.randn((rows, d), generator=g).to(workloads.DTYPES[dtype])
    ob = torch.randn((rows, d), generator=g).to(workloads.DTYPES[dtype])
    la = (torch.randn((rows,), generator=g) * 4).float()
    lb = (torch.randn((rows,), generator=g) * 4).float()
    la[::7] = float("-inf")   # empty key set on one side
    lb[3::11] = float("-inf")
    lb[::77] = float("-inf")  # some rows empty on both sides
    la[::77] = float("-inf")
    return oa, la, ob, lb


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rows", [1, 77, 1000, 4099])
def test_merge_lse(dtype, d, rows):
    oa, la, ob, lb = merge_inputs(rows, d, dtype, zlib.crc32(repr((dtype, d, rows)).encode()))
    a, al, b, bl = to_dev(oa, la, ob, lb)
    o, lse = fa.fa_merge_lse(a, al, b, bl)
    torch.cuda.synchronize()
    ro, rl = oracle.merge_lse(oa, la, ob, lb)
    og, lg = f64(o), f64(lse)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lg), fin)
    assert np.all(og[~fin] == 0)
    err = np.abs(og - ro)[fin]
    assert np.all(err <= REL[dtype] * np.abs(ro[fin]) + 2e-6 * np.abs(ro).max()), err.max()
    assert np.all(np.abs(lg[fin] - rl[fin]) <= 4 * 2.0 ** -24 * np.maximum(1, np.abs(rl[fin])))
    # in place into the first side: bitwise the same
    fa.fa_merge_lse(a, al, b, bl, out=a, lse=al)
    torch.cuda.synchronize()
    assert torch.equal(a, o) and torch.equal(al, lse)


def run_mm(inp, mode=fa.FA_MULTIMODAL_SPLIT_MERGE):
    names = ("q_img", "k_img", "v_img", "q_txt", "k_txt", "v_txt")
    dev = to_dev(*(inp[n] for n in names))
    d = inp["q_img"].shape[-1]
    out = fa.fa_multimodal_forward(*dev, workloads.default_scale(d), text_mode=mode)
    torch.cuda.synchronize()
    return out, dev


SHAPES = [(1, 1, 1, 1), (2, 2, 9, 14), (1, 3, 576, 300), (1, 2, 130, 257), (1, 1, 64, 1),
          (1, 2, 1, 200)]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_multimodal_small(dtype, d, shape):
    B, H, ni, nt = shape
    seed = zlib.crc32(repr(("mm", dtype, d, shape)).encode()) % 100000
    inp = workloads.gen_multimodal(B, H, ni, nt, d, dtype, seed)
    (oi, li, ot, lt), dev = run_mm(inp)
    scale = workloads.default_scale(d)
    roi, rli, rot, rlt = oracle.multimodal(inp["q_img"], inp["k_img"], inp["v_img"],
                                           inp["q_txt"], inp["k_txt"], inp["v_txt"], scale)
    check(oi, li, roi, rli, dtype, f"image {dtype} d{d} {shape}")
    check(ot, lt, rot, rlt, dtype, f"text {dtype} d{d} {shape}")
    # one prefix-LM call over [image; text]: the same attention
    q, k, v = (torch.cat([dev[i], dev[i + 3]], dim=2).contiguous() for i in range(3))
    o1, l1 = fa.fa_forward(q, k, v, scale, fa.FA_MASK_PREFIX_LM, 0, ni)
    torch.cuda.synchronize()
    check(oi, li, f64(o1[:, :, :ni]), f64(l1[:, :, :ni]), dtype, "image vs one call")
    check(ot, lt, f64(o1[:, :, ni:]), f64(l1[:, :, ni:]), dtype, "text vs one call")


FUSED_SHAPES = [(1, 1, 64, 1), (2, 2, 32, 50), (1, 3, 576, 300), (1, 2, 128, 257),
                (1, 2, 96, 33), (1, 1, 32, 1000)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("shape", FUSED_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_multimodal_fused_small(dtype, d, shape):
    """Fused text call (keys read from the image and the text tensors in one launch) against
    the oracle, and against the article's three-call split with its merge."""
    B, H, ni, nt = shape
    seed = zlib.crc32(repr(("mmf", dtype, d, shape)).encode()) % 100000
    inp = workloads.gen_multimodal(B, H, ni, nt, d, dtype, seed)
    (oi, li, ot, lt), _ = run_mm(inp, fa.FA_MULTIMODAL_FUSED)
    scale = workloads.default_scale(d)
    roi, rli, rot, rlt = oracle.multimodal(inp["q_img"], inp["k_img"], inp["v_img"],
                                           inp["q_txt"], inp["k_txt"], inp["v_txt"], scale)
    check(oi, li, roi, rli, dtype, f"fused image {dtype} d{d} {shape}")
    check(ot, lt, rot, rlt, dtype, f"fused text {dtype} d{d} {shape}")
    (si, sli, so, slt), _ = run_mm(inp, fa.FA_MULTIMODAL_SPLIT_MERGE)
    assert torch.equal(oi, si) and torch.equal(li, sli)  # the image call is the same launch
    check(ot, lt, f64(so), f64(slt), dtype, "fused text vs split")


def test_multimodal_full_size():
    """Every element of the multimodal workload, split-merge and fused text modes."""
    w, inp = workloads.gen_workload("multimodal_bf16")
    (oi, li, ot, lt), _ = run_mm(inp)
    (fi, fli, fo, flt), _ = run_mm(inp, fa.FA_MULTIMODAL_FUSED)
    scale = workloads.default_scale(w["d"])
    roi, rli, rot, rlt = oracle.multimodal(inp["q_img"], inp["k_img"], inp["v_img"],
                                           inp["q_txt"], inp["k_txt"], inp["v_txt"], scale)
    check(oi, li, roi, rli, "bf16", "image")
    check(ot, lt, rot, rlt, "bf16", "text")
    check(fi, fli, roi, rli, "bf16", "fused image")
    check(fo, flt, rot, rlt, "bf16", "fused text")