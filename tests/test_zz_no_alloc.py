"""fa_decode_paged_noalloc (the decode entry point that allocates nothing: its split partials
live in the library's static scratch array) against fa_decode_paged with a caller workspace,
through the C ABI on the GPU: two calls in a row, the second smaller, each equal bit for bit
to the workspace entry point (same kernels, same split) and within the forward tolerances of
the fp64 oracle."""
import pytest
import torch

import oracle
import tiled_exact_attention_forward_amd as fa
import workloads
from gpu_util import check, to_dev

pytestmark = pytest.mark.gpu


def run_both(inp, scale):
    q, kp, vp, pt, sl = to_dev(inp["q"], inp["k_pages"], inp["v_pages"], inp["page_table"],
                               inp["seq_lens"])
    S, H, d = q.shape
    o1 = torch.full_like(q, 3.0)
    l1 = torch.full((S, H), 3.0, dtype=torch.float32, device=q.device)
    fa.fa_decode_paged_noalloc(q, kp, vp, pt, sl, scale, out=o1, lse=l1)
    torch.cuda.synchronize()
    o2, l2 = fa.fa_decode_paged(q, kp, vp, pt, sl, scale)
    torch.cuda.synchronize()
    return o1, l1, o2, l2


def test_noalloc_decode_two_calls_second_smaller():
    scale = workloads.default_scale(128)
    _, big = workloads.gen_workload("decode_f16")
    _, small = workloads.gen_workload("decode_f16", S=3, H=16, lens=[300, 1, 2049],
                                      max_len=4096)
    for label, inp in (("decode_f16", big), ("small", small)):
        o1, l1, o2, l2 = run_both(inp, scale)
        assert torch.equal(o1, o2), label
        assert torch.equal(l1, l2), label
        ro, rl = oracle.decode_paged(inp["q"], inp["k_pages"], inp["v_pages"],
                                     inp["page_table"], inp["seq_lens"], scale)
        check(o1, l1, ro, rl, "f16", label)
