"""The benchmark's byte and FLOP accounting against the numbers the pages print and against
the oracle's own count of visible keys."""
import json
import math
import os

import numpy as np
import pytest

import bench
import oracle
import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_arithmetic.json")


def test_page_printed_byte_counts():
    g = json.load(open(GOLDEN))
    s = g["score_matrix_bytes"]
    assert bench.score_matrix_bytes(s["B"], s["H"], s["N"], s["elem_bytes"]) == s["bytes"]
    assert abs(s["bytes"] / 1e9 - 8) < 0.6  # the page rounds to "8GB"
    t = g["fp16_tile_bytes"]
    assert bench.tile_bytes(t["rows"], t["cols"], t["elem_bytes"]) == t["bytes"] == 32 * 1024
    t3 = g["three_tiles_bytes"]
    assert bench.tile_bytes(t3["rows"], t3["cols"], t3["elem_bytes"], t3["tiles"]) == t3["bytes"]
    sp = g["sequence_shard_tokens"]
    assert sp["seq_len"] // sp["shards"] == sp["tokens"]


@pytest.mark.parametrize("Nq,Nkv,mode,W,G", [(64, 64, 0, 0, 0), (64, 64, 1, 0, 0),
                                              (40, 90, 1, 0, 0), (90, 40, 1, 0, 0),
                                              (120, 120, 2, 16, 5), (70, 150, 2, 33, 60),
                                              (50, 50, 2, 1, 0), (50, 50, 2, 200, 0),
                                              (80, 80, 3, 7, 0), (40, 90, 3, 5, 0),
                                              (90, 40, 3, 0, 0), (80, 80, 4, 0, 20),
                                              (40, 90, 4, 0, 60), (90, 40, 4, 0, 5)])
def test_visible_counts_match_oracle(Nq, Nkv, mode, W, G):
    q = np.zeros((1, 1, Nq, 4), np.float32)
    k = np.random.default_rng(0).standard_normal((1, 1, Nkv, 4)).astype(np.float32)
    _, lse = oracle.attention(q, k, k, 1.0, mode, W, G)
    from_oracle = np.where(np.isneginf(lse[0, 0]), 0, np.rint(np.exp(lse[0, 0]))).astype(np.int64)
    assert np.array_equal(bench.visible_counts(Nq, Nkv, mode, W, G), from_oracle)
    assert np.array_equal(bench.visible_counts(Nq, Nkv, mode, W, G),
                          [len(pins.visible_keys(i + Nkv - Nq, Nkv, mode, W, G)) for i in range(Nq)])


def test_workload_flop_counts():
    import workloads
    f, pairs = bench.prefill_flops(workloads.WORKLOADS["dense_bf16"])
    assert f == 4 * 128 * 4 * 32 * 1024 * 1024 == 68719476736
    _, pairs = bench.prefill_flops(workloads.WORKLOADS["window_bf16"])
    assert pairs == 32 * 66976800
    _, pairs = bench.prefill_flops(workloads.WORKLOADS["causal_bf16"])
    assert pairs == 4 * 32 * 4096 * 4097 // 2


def test_paged_prefill_pair_count():
    """Chunk row i of a sequence with L keys and an n-token chunk sees i + L - n + 1 keys
    (causal); the count is checked against the closed form summed over the chunk."""
    w = dict(mask=1, window=0, n_global=0, H=3)
    lens, qls = [700, 256, 1], [300, 0, 1]
    want = 3 * sum(sum(i + L - n + 1 for i in range(n)) for L, n in zip(lens, qls))
    assert bench.paged_prefill_pairs(w, lens, qls) == want


def test_multimodal_pair_count():
    """Image rows see the image; text rows see the image and earlier text: the same count
    as the prefix-LM mask over [image; text] with the image as prefix."""
    w = dict(n_img=5, n_txt=7, B=2, H=3)
    want = int(bench.visible_counts(12, 12, 4, 0, 5).sum()) * 6
    assert bench.multimodal_pairs(w) == want
