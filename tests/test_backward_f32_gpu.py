"""The float32 backward (fa_backward with FA_F32 through the C ABI) against the fp64 oracle's
gradients, beyond the small shapes that test_backward_gpu and test_backward_block_sparse_gpu
run for every dtype: larger shapes with every element compared, a negative scale with inputs
large enough to make P nearly one-hot, scale 0, and bitwise reproducibility. Tolerance:
check_grads with u = 2^-16 (derived in gpu_util).
"""
import pytest
import torch

import oracle
import tiled_exact_attention_forward_amd as fa
import workloads
from gpu_util import check_grads, to_dev
from pins import band_mask

pytestmark = pytest.mark.gpu


def run_bwd(q, k, v, do, scale, mask=0, W=0, G=0):
    qd, kd, vd, gd = to_dev(q, k, v, do)
    o, lse = fa.fa_forward(qd, kd, vd, scale, mask, W, G)
    dq, dk, dv = fa.fa_backward(qd, kd, vd, o, lse, gd, scale, mask, W, G)
    torch.cuda.synchronize()
    assert dq.dtype == torch.float32
    return dq, dk, dv


@pytest.mark.parametrize("mask", [(0, 0, 0), (1, 0, 0), (2, 300, 16), (3, 100, 0), (4, 0, 900)],
                         ids=lambda m: f"m{m[0]}w{m[1]}g{m[2]}")
def test_backward_f32_larger(mask):
    """B2 H4, 1000 query rows against 1500 keys (ragged tails on both), d 128: every element."""
    q, k, v = workloads.gen_prefill(2, 4, 1000, 1500, 128, "f32", 61)
    do = workloads.gen_dout((2, 4, 1000, 128), "f32", 62)
    scale = workloads.default_scale(128)
    got = run_bwd(q, k, v, do, scale, *mask)
    ref = oracle.attention_backward(q, k, v, do, scale, *mask)
    e = check_grads(got, ref, "f32", f"f32 mask {mask}", (q, k, v, do), scale,
                    band_mask(1000, 1500, *mask))
    print("f32 backward", mask, e)


def test_backward_f32_negative_scale_and_large_inputs():
    q, k, v = workloads.gen_prefill(1, 2, 200, 300, 64, "f32", 63, input_scale=8.0)
    do = workloads.gen_dout((1, 2, 200, 64), "f32", 64)
    for scale in (-workloads.default_scale(64), workloads.default_scale(64)):
        for mask in ((0, 0, 0), (1, 0, 0), (3, 20, 0)):
            got = run_bwd(q, k, v, do, scale, *mask)
            ref = oracle.attention_backward(q, k, v, do, scale, *mask)
            check_grads(got, ref, "f32", f"scale {scale} mask {mask}", (q, k, v, do), scale,
                        band_mask(200, 300, *mask))


def test_backward_f32_zero_scale():
    """scale 0 makes P uniform over each row's visible keys: dQ = dK = 0 exactly."""
    q, k, v = workloads.gen_prefill(1, 2, 100, 150, 128, "f32", 65)
    do = workloads.gen_dout((1, 2, 100, 128), "f32", 66)
    for mask in ((0, 0, 0), (1, 0, 0), (2, 20, 3), (3, 10, 0)):
        got = run_bwd(q, k, v, do, 0.0, *mask)
        ref = oracle.attention_backward(q, k, v, do, 0.0, *mask)
        check_grads(got, ref, "f32", f"scale 0 mask {mask}", (q, k, v, do), 0.0,
                    band_mask(100, 150, *mask))
        assert torch.all(got[0] == 0) and torch.all(got[1] == 0)


def test_backward_f32_deterministic():
    q, k, v = workloads.gen_prefill(2, 2, 640, 700, 128, "f32", 67)
    do = workloads.gen_dout((2, 2, 640, 128), "f32", 68)
    a = run_bwd(q, k, v, do, 0.0884, 1)
    b = run_bwd(q, k, v, do, 0.0884, 1)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
