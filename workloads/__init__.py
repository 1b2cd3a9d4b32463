"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module only draws random numbers and lays them out; it holds none of the attention
arithmetic. Both the HIP path and the oracle consume exactly the tensors it returns.

Recipe (every draw from one torch CPU generator seeded per workload):
  * prefill: Q, K, V drawn in that order as float32 standard normals of shape [B,H,N,d],
    optionally multiplied by an exact power of two in float32, then cast to the run's dtype
    (round to nearest even);
  * backward: dO [B,H,Nq,d] from its own generator (gen_dout), float32 standard normals
    cast to the run's dtype;
  * chunked prefill (paged): Q [S,Qmax,H,d] (rows past each chunk NaN), the chunk lengths,
    then a seed for the paged cache, drawn like decode's;
  * multimodal: the image's Q, K, V like prefill with the workload seed, then the text's
    with seed + 1;
  * paged decode: Q [S,H,d], then the S sequence lengths uniform in [len_lo, len_hi], then a
    random permutation of the physical page ids, then the K and V page pools
    [num_pages, page_size, H, d]. Slots past a sequence's length in its last page and the
    spare pages hold NaN, so a kernel that reads them without masking shows it.

The workloads stand in for the shapes the pages report (the pages' LLaMA-7B, BERT and long
document runs need weights and datasets that are not used here).
"""
import math

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# name -> workload description. mask: 0 none, 1 causal, 2 causal sliding window + global keys,
# 3 band of `window` positions on both sides, 4 prefix LM with an `n_global`-key prefix,
# 5 block sparse (a seeded layout of block x block tiles, see gen_layout).
WORKLOADS = {
    "tiny_f32": dict(kind="prefill", B=1, H=2, Nq=128, Nkv=128, d=64, dtype="f32", mask=0,
                     window=0, n_global=0, input_scale=1.0, seed=1),
    "dense_f16": dict(kind="prefill", B=4, H=32, Nq=1024, Nkv=1024, d=128, dtype="f16",
                      mask=0, window=0, n_global=0, input_scale=1.0, seed=2),
    "dense_bf16": dict(kind="prefill", B=4, H=32, Nq=1024, Nkv=1024, d=128, dtype="bf16",
                       mask=0, window=0, n_global=0, input_scale=1.0, seed=2),
    "dense_f32": dict(kind="prefill", B=4, H=32, Nq=1024, Nkv=1024, d=128, dtype="f32",
                      mask=0, window=0, n_global=0, input_scale=1.0, seed=2),
    "causal_bf16": dict(kind="prefill", B=4, H=32, Nq=4096, Nkv=4096, d=128, dtype="bf16",
                        mask=1, window=0, n_global=0, input_scale=0.5, seed=3),
    "window_bf16": dict(kind="prefill", B=1, H=32, Nq=32768, Nkv=32768, d=128, dtype="bf16",
                        mask=2, window=2048, n_global=64, input_scale=1.0, seed=4),
    "band_bf16": dict(kind="prefill", B=1, H=32, Nq=32768, Nkv=32768, d=128, dtype="bf16",
                      mask=3, window=2048, n_global=0, input_scale=1.0, seed=6),
    "prefix_bf16": dict(kind="prefill", B=4, H=32, Nq=4096, Nkv=4096, d=128, dtype="bf16",
                        mask=4, window=0, n_global=1024, input_scale=0.5, seed=7),
    "blocksparse_bf16": dict(kind="prefill", B=1, H=32, Nq=16384, Nkv=16384, d=128,
                             dtype="bf16", mask=5, window=0, n_global=0, input_scale=1.0,
                             seed=8, block=128, density=0.125),
    "prefill_paged_bf16": dict(kind="prefill_paged", S=8, Qmax=1024, H=32, d=128,
                               dtype="bf16", page_size=256, len_lo=4096, len_hi=8192,
                               max_len=8192, q_lo=512, q_hi=1024, spare_pages=4, mask=1,
                               window=0, n_global=0, seed=9),
    "multimodal_bf16": dict(kind="multimodal", B=4, H=32, n_img=576, n_txt=2048, d=128,
                            dtype="bf16", input_scale=1.0, seed=10),
    "decode_f16": dict(kind="decode", S=8, H=32, d=128, dtype="f16", page_size=256,
                       len_lo=4096, len_hi=8192, max_len=8192, spare_pages=4, seed=5),
}


def default_scale(d):
    """The float32 value of 1/sqrt(d) that both sides receive."""
    return float(np.float32(1.0 / math.sqrt(d)))


def gen_prefill(B, H, Nq, Nkv, d, dtype, seed, input_scale=1.0):
    """Q [B,H,Nq,d], K and V [B,H,Nkv,d] on the CPU in `dtype` ("f32", "f16", "bf16")."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    q = torch.randn((B, H, Nq, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, H, Nkv, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, H, Nkv, d), generator=g, dtype=torch.float32)
    if input_scale != 1.0:
        q.mul_(input_scale)
        k.mul_(input_scale)
        v.mul_(input_scale)
    t = DTYPES[dtype]
    return q.to(t), k.to(t), v.to(t)


def gen_dout(shape, dtype, seed, input_scale=1.0):
    """Upstream gradient dO for the backward pass: float32 standard normals of `shape` from a
    generator seeded `seed` (its own stream, so Q, K, V stay those of the forward),
    optionally times an exact power of two, cast to `dtype`."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    do = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if input_scale != 1.0:
        do.mul_(input_scale)
    return do.to(DTYPES[dtype])


def gen_layout(H, Nq, Nkv, block, density, seed):
    """Block-sparse layout [H, ceil(Nq/block), ceil(Nkv/block)] uint8: each tile visible with
    probability `density` (one uniform draw per tile from a generator seeded `seed`), plus
    the diagonal tiles, so that every query block sees at least one key block when
    Nkv >= Nq."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    nqb, nkb = -(-Nq // block), -(-Nkv // block)
    lay = (torch.rand((H, nqb, nkb), generator=g) < density).to(torch.uint8)
    n = min(nqb, nkb)
    lay[:, torch.arange(n), torch.arange(n)] = 1
    return lay


def gen_decode(S, H, d, dtype, seed, page_size=256, len_lo=4096, len_hi=8192, max_len=None,
               spare_pages=4, lens=None):
    """Paged decode inputs.

    Returns dict with q [S,H,d], k_pages/v_pages [P,page_size,H,d] (dtype), page_table
    [S,max_pages] int32 (-1 where unused), seq_lens [S] int32. `lens` overrides the drawn
    lengths (the draw still happens so the rest of the stream is unchanged).
    """
    g = torch.Generator("cpu").manual_seed(int(seed))
    t = DTYPES[dtype]
    q = torch.randn((S, H, d), generator=g, dtype=torch.float32)
    drawn = torch.randint(len_lo, len_hi + 1, (S,), generator=g, dtype=torch.int64)
    L = drawn if lens is None else torch.as_tensor(lens, dtype=torch.int64)
    if max_len is None:
        max_len = int(L.max())
    max_pages = (max_len + page_size - 1) // page_size
    pages_per_seq = [(int(x) + page_size - 1) // page_size for x in L]
    assert max(pages_per_seq) <= max_pages
    used = sum(pages_per_seq)
    total = used + int(spare_pages)
    perm = torch.randperm(total, generator=g)
    k_pages = torch.randn((total, page_size, H, d), generator=g, dtype=torch.float32)
    v_pages = torch.randn((total, page_size, H, d), generator=g, dtype=torch.float32)
    page_table = torch.full((S, max_pages), -1, dtype=torch.int32)
    nxt = 0
    nan = float("nan")
    for s in range(S):
        for p in range(pages_per_seq[s]):
            pid = int(perm[nxt])
            nxt += 1
            page_table[s, p] = pid
        tail = int(L[s]) - (pages_per_seq[s] - 1) * page_size
        last = int(page_table[s, pages_per_seq[s] - 1])
        k_pages[last, tail:] = nan
        v_pages[last, tail:] = nan
    for i in range(used, total):
        k_pages[int(perm[i])] = nan
        v_pages[int(perm[i])] = nan
    return dict(q=q.to(t), k_pages=k_pages.to(t), v_pages=v_pages.to(t),
                page_table=page_table, seq_lens=L.to(torch.int32), page_size=page_size,
                max_pages=max_pages)


def gen_prefill_paged(S, Qmax, H, d, dtype, seed, page_size=256, len_lo=4096, len_hi=8192,
                      max_len=None, q_lo=1, q_hi=None, spare_pages=4, lens=None, qlens=None):
    """Chunked prefill inputs: the paged cache of gen_decode (same recipe and NaN poisoning)
    plus a chunk per sequence. Draw order: Q [S,Qmax,H,d], then the S chunk lengths uniform
    in [q_lo, min(q_hi, Qmax)] (each then capped at its sequence length), then the paged
    cache exactly as gen_decode draws it. Q rows at or past a sequence's chunk hold NaN.
    `lens`/`qlens` override the drawn lengths (the draws still happen)."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    t = DTYPES[dtype]
    q = torch.randn((S, Qmax, H, d), generator=g, dtype=torch.float32)
    hi = Qmax if q_hi is None else min(q_hi, Qmax)
    qdrawn = torch.randint(q_lo, hi + 1, (S,), generator=g, dtype=torch.int64)
    cache = gen_decode(S, H, d, dtype, int(torch.randint(0, 2 ** 31 - 1, (1,), generator=g)),
                       page_size, len_lo, len_hi, max_len, spare_pages, lens)
    L = cache["seq_lens"].to(torch.int64)
    ql = qdrawn if qlens is None else torch.as_tensor(qlens, dtype=torch.int64)
    ql = torch.minimum(ql, L)
    for s in range(S):
        q[s, int(ql[s]):] = float("nan")
    cache["q"] = q.to(t)
    cache["q_lens"] = ql.to(torch.int32)
    return cache


def gen_multimodal(B, H, n_img, n_txt, d, dtype, seed, input_scale=1.0):
    """Image and text attention inputs: the image's Q, K, V [B,H,n_img,d] drawn like
    gen_prefill with `seed`, then the text's Q, K, V [B,H,n_txt,d] with seed + 1."""
    qi, ki, vi = gen_prefill(B, H, n_img, n_img, d, dtype, seed, input_scale)
    qt, kt, vt = gen_prefill(B, H, n_txt, n_txt, d, dtype, seed + 1, input_scale)
    return dict(q_img=qi, k_img=ki, v_img=vi, q_txt=qt, k_txt=kt, v_txt=vt)


def gen_workload(name, **override):
    """Inputs of a named workload (overrides replace any field, e.g. a smaller N)."""
    w = dict(WORKLOADS[name])
    w.update(override)
    if w["kind"] == "prefill":
        q, k, v = gen_prefill(w["B"], w["H"], w["Nq"], w["Nkv"], w["d"], w["dtype"], w["seed"],
                              w.get("input_scale", 1.0))
        out = dict(q=q, k=k, v=v)
        if w["mask"] == 5:  # block sparse: the layout comes after the tensors, own seed
            out["layout"] = gen_layout(w["H"], w["Nq"], w["Nkv"], w["block"], w["density"],
                                       w["seed"] + 1000)
        return w, out
    if w["kind"] == "multimodal":
        return w, gen_multimodal(w["B"], w["H"], w["n_img"], w["n_txt"], w["d"], w["dtype"],
                                 w["seed"], w.get("input_scale", 1.0))
    if w["kind"] == "prefill_paged":
        inp = gen_prefill_paged(w["S"], w["Qmax"], w["H"], w["d"], w["dtype"], w["seed"],
                                w["page_size"], w["len_lo"], w["len_hi"], w.get("max_len"),
                                w.get("q_lo", 1), w.get("q_hi"), w.get("spare_pages", 4),
                                w.get("lens"), w.get("qlens"))
        return w, inp
    inp = gen_decode(w["S"], w["H"], w["d"], w["dtype"], w["seed"], w["page_size"],
                     w["len_lo"], w["len_hi"], w.get("max_len"), w.get("spare_pages", 4),
                     w.get("lens"))
    return w, inp
