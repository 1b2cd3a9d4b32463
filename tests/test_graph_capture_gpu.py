"""The library's calls enqueue only kernel launches on the caller's stream (no allocation, no
memset, no host synchronisation), so a serving loop can capture them into a HIP graph
(torch.cuda.CUDAGraph) and replay it. One graph holds a causal forward with its backward, a
paged decode and a chunked prefill against the same cache; every replay is compared bit for
bit with the eager results on the same inputs, with eager library calls and synchronisations
between the replays, and with the inputs rewritten in place between replays (the graph must
read the current contents of its buffers). A second graph holds the fp32 forward and backward
and the block-sparse forward and backward.
"""
import pytest
import torch

import tiled_exact_attention_forward_amd as fa
import workloads
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


def test_capture_and_replay():
    dev = require_gpu()
    scale = workloads.default_scale(128)
    q, k, v = (t.to(dev) for t in workloads.gen_prefill(1, 4, 500, 500, 128, "bf16", 51))
    do = workloads.gen_dout((1, 4, 500, 128), "bf16", 52).to(dev)
    _, dec = workloads.gen_workload("decode_f16", S=3, H=8, lens=[300, 1000, 2049])
    dq_in, dkp, dvp, dpt, dsl = (dec[x].to(dev) for x in ("q", "k_pages", "v_pages",
                                                            "page_table", "seq_lens"))
    pre = workloads.gen_prefill_paged(2, 300, 4, 128, "bf16", 53, max_len=1000,
                                      lens=[333, 1000], qlens=[70, 300])
    pq, pkp, pvp, ppt, psl, pql = (pre[x].to(dev) for x in ("q", "k_pages", "v_pages",
                                                            "page_table", "seq_lens", "q_lens"))

    # static outputs and workspaces, allocated before the capture
    o, lse = torch.empty_like(q), torch.empty((1, 4, 500), dtype=torch.float32, device=dev)
    gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bws = torch.empty((fa.fa_backward_workspace_bytes(1, 4, 500),), dtype=torch.uint8,
                      device=dev)
    od, ld = torch.empty_like(dq_in), torch.empty((3, 8), dtype=torch.float32, device=dev)
    dws = torch.empty((fa.fa_decode_paged_workspace_bytes(3, 8, 128, dpt.shape[1]),),
                      dtype=torch.uint8, device=dev)
    op = torch.full_like(pq, 7.0)
    lp = torch.full((2, 300, 4), 7.0, dtype=torch.float32, device=dev)

    def calls():
        fa.fa_forward(q, k, v, scale, fa.FA_MASK_CAUSAL, out=o, lse=lse)
        fa.fa_backward(q, k, v, o, lse, do, scale, fa.FA_MASK_CAUSAL, dq=gq, dk=gk, dv=gv,
                       workspace=bws)
        fa.fa_decode_paged(dq_in, dkp, dvp, dpt, dsl, scale, out=od, lse=ld, workspace=dws)
        fa.fa_prefill_paged(pq, pkp, pvp, ppt, psl, pql, scale, out=op, lse=lp)

    outs = (o, lse, gq, gk, gv, od, ld, op, lp)

    def eager():
        calls()
        torch.cuda.synchronize()
        return [t.clone() for t in outs]

    want = eager()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the side stream, as torch recommends
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()

    q2 = workloads.gen_prefill(1, 4, 500, 500, 128, "bf16", 54)[0].to(dev)
    q_orig = q.clone()
    for rep in range(4):
        for t in outs:
            t.fill_(3.0)  # stale values the replay must overwrite
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("o", "lse", "dq", "dk", "dv", "decode o", "decode lse",
                                   "prefill o", "prefill lse"), outs, want):
            if name.startswith("prefill"):  # rows past each chunk keep what was there
                n = (70, 300)
                for si, nq in enumerate(n):
                    assert torch.equal(got[si, :nq], ref[si, :nq]), (rep, name, si)
            else:
                assert torch.equal(got, ref), (rep, name)
        # eager work between replays, then new inputs written in place for the next replay
        fa.fa_forward(q2, k, v, scale, fa.FA_MASK_NONE)
        torch.cuda.synchronize()
        q.copy_(q2 if rep % 2 == 0 else q_orig)
        want = eager()


def test_capture_fp32_and_block_sparse():
    """The fp32 forward and backward and the block-sparse forward and backward in one graph,
    replayed against eager results as above."""
    dev = require_gpu()
    scale = workloads.default_scale(64)
    q, k, v = (t.to(dev) for t in workloads.gen_prefill(2, 2, 300, 450, 64, "f32", 55))
    do = workloads.gen_dout((2, 2, 300, 64), "f32", 56).to(dev)
    bq, bk, bv = (t.to(dev) for t in workloads.gen_prefill(1, 2, 300, 450, 128, "bf16", 57))
    bdo = workloads.gen_dout((1, 2, 300, 128), "bf16", 58).to(dev)
    g = torch.Generator("cpu").manual_seed(59)
    lay = (torch.rand((2, 3, 4), generator=g) < 0.5).to(torch.uint8).to(dev)

    o, lse = torch.empty_like(q), torch.empty((2, 2, 300), dtype=torch.float32, device=dev)
    gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty((fa.fa_backward_workspace_bytes(2, 2, 300),), dtype=torch.uint8,
                     device=dev)
    bo, blse = torch.empty_like(bq), torch.empty((1, 2, 300), dtype=torch.float32, device=dev)
    bgq, bgk, bgv = torch.empty_like(bq), torch.empty_like(bk), torch.empty_like(bv)
    bws = torch.empty((fa.fa_backward_workspace_bytes(1, 2, 300),), dtype=torch.uint8,
                      device=dev)

    def calls():
        fa.fa_forward(q, k, v, scale, fa.FA_MASK_BAND, 40, out=o, lse=lse)
        fa.fa_backward(q, k, v, o, lse, do, scale, fa.FA_MASK_BAND, 40, dq=gq, dk=gk, dv=gv,
                       workspace=ws)
        fa.fa_forward_block_sparse(bq, bk, bv, lay, 128, scale, out=bo, lse=blse)
        fa.fa_backward_block_sparse(bq, bk, bv, bo, blse, bdo, lay, 128, scale, dq=bgq, dk=bgk,
                                    dv=bgv, workspace=bws)

    outs = (o, lse, gq, gk, gv, bo, blse, bgq, bgk, bgv)
    calls()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.fill_(3.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (got, ref) in enumerate(zip(outs, want)):
            assert torch.equal(got, ref), (rep, i)
        fa.fa_forward(q, k, v, scale, fa.FA_MASK_NONE)  # eager work between replays
        torch.cuda.synchronize()
