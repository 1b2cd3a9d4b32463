"""Parity of chunked prefill against a paged cache (fa_prefill_paged, through the C ABI) with
the fp64 oracle, on the GPU.

Each sequence's chunk (its newest q_lens[s] tokens) attends to its seq_lens[s] cached keys
with bottom-right masks. Small cases compare every row of every chunk across ragged page
tails, empty chunks, one-token chunks and whole-sequence chunks, with head counts that are
and are not multiples of 8 (the two work placements); the full-size chunked prefill
workload compares every row of every (sequence, head) pair. Histories past 64 pages
(16,384 keys) take the kernel's reload of the page ids. Unused page slots and spare
pages hold NaN, and Q rows past each chunk hold NaN, so reading any of them shows. Rows past
a chunk must be left as they were. Tolerances are those of the forward (gpu_util).
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

SENT = 7.0  # sentinel in rows no chunk covers


def run_prefill(inp, scale, mask=(1, 0, 0)):
    q, kp, vp, pt, sl, ql = to_dev(inp["q"], inp["k_pages"], inp["v_pages"],
                                   inp["page_table"], inp["seq_lens"], inp["q_lens"])
    S, Qmax, H, d = q.shape
    out = torch.full_like(q, SENT)
    lse = torch.full((S, Qmax, H), SENT, dtype=torch.float32, device=q.device)
    fa.fa_prefill_paged(q, kp, vp, pt, sl, ql, scale, *mask, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def compare(out, lse, ro, rl, q_lens, dtype, label):
    og, lg = out.cpu(), lse.cpu()
    for s, nq in enumerate(int(x) for x in q_lens):
        assert torch.all(og[s, nq:] == SENT) and torch.all(lg[s, nq:] == SENT), \
            f"{label}: rows past chunk {s} were written"
        if nq:
            check(og[s, :nq], lg[s, :nq], ro[s, :nq], rl[s, :nq], dtype, f"{label} seq {s}")


MASKS = [(1, 0, 0), (0, 0, 0), (2, 100, 5), (2, 300, 64), (3, 50, 0), (4, 0, 70)]
CASES = [  # (seq_lens, q_lens, Qmax)
    ([1, 16, 255, 256, 257, 700], [1, 16, 100, 256, 129, 300], 300),
    ([513, 1000, 77, 300], [0, 1, 77, 33], 128),
    ([2048, 1500], [600, 1500], 1500),
]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", MASKS, ids=lambda m: f"m{m[0]}w{m[1]}g{m[2]}")
@pytest.mark.parametrize("case", range(len(CASES)))
def test_prefill_paged_small(dtype, d, mask, case):
    lens, qls, Qmax = CASES[case]
    seed = zlib.crc32(repr(("pre", dtype, d, mask, case)).encode()) % 100000
    H = 4 if d == 64 else 2
    inp = workloads.gen_prefill_paged(len(lens), Qmax, H, d, dtype, seed, max_len=max(lens),
                                      lens=lens, qlens=qls)
    scale = workloads.default_scale(d)
    out, lse = run_prefill(inp, scale, mask)
    ro, rl = oracle.prefill_paged(inp["q"], inp["k_pages"], inp["v_pages"], inp["page_table"],
                                  inp["seq_lens"], inp["q_lens"], scale, *mask)
    compare(out, lse, ro, rl, inp["q_lens"], dtype, f"{dtype} d{d} mask{mask} case{case}")


@pytest.mark.parametrize("mask", [(1, 0, 0), (2, 100, 5), (4, 0, 70)])
def test_prefill_paged_matches_contiguous_forward(mask):
    """The paged kernel is the forward kernel with paged addressing: on the same values a
    chunk gives bitwise the results of fa_forward on the contiguous keys."""
    lens, qls = [700, 257, 1024], [300, 257, 1]
    inp = workloads.gen_prefill_paged(3, 300, 4, 128, "bf16", 4321, max_len=1024, lens=lens,
                                      qlens=qls)
    scale = workloads.default_scale(128)
    out, lse = run_prefill(inp, scale, mask)
    kp, vp, pt = inp["k_pages"], inp["v_pages"], inp["page_table"]
    for s, (L, nq) in enumerate(zip(lens, qls)):
        idx = torch.arange(L)
        rows = pt[s, idx // 256].long() * 256 + idx % 256
        k = kp.reshape(-1, 4, 128)[rows].permute(1, 0, 2)[None].contiguous()
        v = vp.reshape(-1, 4, 128)[rows].permute(1, 0, 2)[None].contiguous()
        q = inp["q"][s, :nq].permute(1, 0, 2)[None].contiguous()
        qd, kd, vd = to_dev(q, k, v)
        o2, l2 = fa.fa_forward(qd, kd, vd, scale, *mask)
        torch.cuda.synchronize()
        assert torch.equal(out[s, :nq], o2[0].permute(1, 0, 2)), s
        assert torch.equal(lse[s, :nq], l2[0].permute(1, 0)), s


# Every XCD receives H/8 heads of every sequence when H is a multiple of 8, and pairs in
# another order otherwise: both placements, every row of every chunk compared.
@pytest.mark.parametrize("H", [8, 16, 32])
@pytest.mark.parametrize("mask", [(1, 0, 0), (2, 100, 5)], ids=lambda m: f"m{m[0]}w{m[1]}g{m[2]}")
def test_prefill_paged_heads_multiple_of_8(H, mask):
    lens, qls = [300, 1, 1000, 513, 257, 64, 700, 129, 900], [300, 1, 200, 0, 257, 33, 129, 100, 1]
    seed = zlib.crc32(repr(("pre8", H, mask)).encode()) % 100000
    inp = workloads.gen_prefill_paged(len(lens), 300, H, 128, "bf16", seed, max_len=1000,
                                      lens=lens, qlens=qls)
    scale = workloads.default_scale(128)
    out, lse = run_prefill(inp, scale, mask)
    ro, rl = oracle.prefill_paged(inp["q"], inp["k_pages"], inp["v_pages"], inp["page_table"],
                                  inp["seq_lens"], inp["q_lens"], scale, *mask)
    compare(out, lse, ro, rl, inp["q_lens"], "bf16", f"H{H} mask{mask}")


@pytest.mark.parametrize("nseq", [63, 64, 65, 70])
def test_prefill_paged_many_sequences(nseq):
    """Up to 64 sequences are placed in order of decreasing work, more keep their index order:
    both sides of that limit, every row of every chunk (lengths drawn per sequence, some
    chunks empty, ties in work)."""
    g = np.random.default_rng(nseq)
    lens = g.integers(1, 700, nseq).tolist()
    qls = [int(min(x, q)) for x, q in zip(lens, g.integers(0, 200, nseq))]
    lens[1], qls[1] = lens[0], qls[0]  # a tie in work
    qls[2] = 0                         # an empty chunk
    inp = workloads.gen_prefill_paged(nseq, 200, 8, 128, "bf16", 1000 + nseq, max_len=700,
                                      lens=lens, qlens=qls)
    # Short sequences give rows that see 1-3 keys, whose outputs are single draws of V. V/4
    # (exact in bf16) keeps |O| < 2: above 2 one bf16 step (2^-6) is wider than the 1e-2 bound.
    inp["v_pages"] = inp["v_pages"] * 0.25
    scale = workloads.default_scale(128)
    out, lse = run_prefill(inp, scale, (1, 0, 0))
    ro, rl = oracle.prefill_paged(inp["q"], inp["k_pages"], inp["v_pages"], inp["page_table"],
                                  inp["seq_lens"], inp["q_lens"], scale, 1, 0, 0)
    compare(out, lse, ro, rl, inp["q_lens"], "bf16", f"{nseq} sequences")


@pytest.mark.parametrize("mask", [(1, 0, 0), (2, 1000, 64), (0, 0, 0)])
def test_prefill_paged_long_history(mask):
    """Histories past 64 pages (16,384 keys), where the kernel loads the next 64 page ids on
    the way; the window mask jumps from the global tokens in page 0 to pages past 64."""
    lens, qls = [20000, 17000, 300], [64, 200, 300]
    inp = workloads.gen_prefill_paged(3, 300, 8, 128, "bf16", 77, max_len=20000, lens=lens,
                                      qlens=qls)
    inp["v_pages"] = inp["v_pages"] * 0.25  # the whole-sequence chunk's first rows: |O| < 2
    scale = workloads.default_scale(128)
    out, lse = run_prefill(inp, scale, mask)
    ro, rl = oracle.prefill_paged(inp["q"], inp["k_pages"], inp["v_pages"], inp["page_table"],
                                  inp["seq_lens"], inp["q_lens"], scale, *mask)
    compare(out, lse, ro, rl, inp["q_lens"], "bf16", f"long history mask {mask}")


@pytest.mark.timeout(600)
def test_prefill_paged_full_size():
    """Every row of every (sequence, head) pair of the chunked-prefill workload; rows past
    each chunk must still hold the sentinel."""
    w, inp = workloads.gen_workload("prefill_paged_bf16")
    scale = workloads.default_scale(w["d"])
    mask = (w["mask"], w["window"], w["n_global"])
    out, lse = run_prefill(inp, scale, mask)
    ro, rl = oracle.prefill_paged(inp["q"], inp["k_pages"], inp["v_pages"], inp["page_table"],
                                  inp["seq_lens"], inp["q_lens"], scale, *mask)
    compare(out, lse, ro, rl, inp["q_lens"], w["dtype"], "prefill_paged_bf16")
