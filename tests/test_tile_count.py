"""The bench's tile-granular work count (bench.tile_elements) against brute force over the
mask definition: a tile counts when any of its (query, key) pairs is visible."""
import numpy as np
import pytest

import bench
from pins import band_mask


@pytest.mark.parametrize("Nq,Nkv", [(1, 1), (100, 100), (300, 257), (129, 700), (256, 256)])
@pytest.mark.parametrize("mode,W,G", [(0, 0, 0), (1, 0, 0), (2, 40, 5), (2, 1, 0), (2, 100, 70),
                                      (3, 0, 0), (3, 33, 0), (4, 0, 70), (4, 0, 0)])
def test_tile_elements_brute_force(Nq, Nkv, mode, W, G):
    vis = band_mask(Nq, Nkv, mode, W, G).numpy()
    tiles = elems = 0
    for i0 in range(0, Nq, 128):
        for k0 in range(0, Nkv, 32):
            blk = vis[i0:i0 + 128, k0:k0 + 32]
            if blk.any():
                tiles += 1
                elems += blk.size
    assert bench.tile_elements(Nq, Nkv, mode, W, G) == (tiles, elems)


def test_tile_elements_block_sparse():
    g = np.random.default_rng(5)
    lay = (g.random((2, 3, 5)) < 0.4).astype(np.uint8)  # H 2, Nq 300 (3 blocks), Nkv 600
    tiles = elems = 0
    for h in range(2):
        for qb in range(3):
            rows = min(128, 300 - 128 * qb)
            for k0 in range(0, 600, 32):
                if lay[h, qb, k0 // 128]:
                    tiles += 1
                    elems += rows * min(32, 600 - k0)
    assert bench.tile_elements(300, 600, 5, layout=lay) == (tiles, elems)
