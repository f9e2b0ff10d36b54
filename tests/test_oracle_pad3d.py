"""Pins of the oracle's 3D-padded layout (one block per tile, padding inside
the sequence) and of the per-block valid counts it feeds to pool / attention."""
import json
import os
from math import sqrt

import numpy as np

from oracle import svsa_oracle as orc


def test_pad3d_hand_worked_layouts(golden_dir=None):
    golden_dir = golden_dir or os.path.join(os.path.dirname(__file__), "golden")
    with open(os.path.join(golden_dir, "pad3d_layout.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        slots, counts = orc.block_layout(tuple(c["grid"]), tuple(c["tile"]), pad3d=True)
        assert slots.tolist() == c["slots"]
        assert counts.tolist() == c["counts"]


def test_pad3d_equals_packed_when_tiles_divide():
    for grid, tile in (((4, 8, 8), (2, 4, 4)), ((8, 16, 16), (4, 4, 4)), ((6, 8, 16), (3, 8, 16))):
        a, ca = orc.block_layout(grid, tile, pad3d=True)
        b, cb = orc.block_layout(grid, tile, pad3d=False)
        assert np.array_equal(a, b) and np.array_equal(ca, cb)


def test_pad3d_blocks_are_whole_tiles_valid_first():
    grid, tile = (5, 7, 9), (2, 4, 4)
    T, H, W = grid
    slots, counts = orc.block_layout(grid, tile, pad3d=True)
    Bk = int(np.prod(tile))
    valid = slots[slots >= 0]
    assert np.array_equal(np.sort(valid), np.arange(T * H * W))
    for k, n in enumerate(counts):
        blk = slots[k * Bk:(k + 1) * Bk]
        assert np.all(blk[:n] >= 0) and np.all(blk[n:] == -1)
        t, rem = np.divmod(blk[:n], H * W)
        h, w = np.divmod(rem, W)
        assert len({(a, b, c) for a, b, c in zip(t // tile[0], h // tile[1], w // tile[2])}) == 1


def test_pad3d_pool_is_the_mean_of_each_tile():
    grid, tile = (5, 7, 9), (2, 4, 4)
    T, H, W = grid
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 2, T * H * W, 8))
    slots, counts = orc.block_layout(grid, tile, pad3d=True)
    xp = orc.permute_fwd(x, grid, tile, pad3d=True)
    got = orc.pool(xp, T * H * W, int(np.prod(tile)), counts)
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    tid = ((t // 2) * 2 + (h // 4)) * 3 + (w // 4)          # tile grid 3 x 2 x 3
    for k in range(len(counts)):
        sel = (tid.ravel() == k)
        assert np.allclose(got[0, :, k], x[0][:, sel].mean(axis=1), rtol=1e-13, atol=1e-13)


def test_pad3d_full_attention_equals_dense():
    grid, tile = (3, 5, 6), (2, 4, 4)
    T, H, W = grid
    N, Bk, D = T * H * W, 32, 16
    rng = np.random.default_rng(8)
    q, k, v = (rng.standard_normal((1, 1, N, D)) for _ in range(3))
    slots, counts = orc.block_layout(grid, tile, pad3d=True)
    nb = len(counts)
    qp, kp, vp = (orc.permute_fwd(a, grid, tile, pad3d=True) for a in (q, k, v))
    kp[:, :, slots < 0] = 1e6            # padding must never be read
    vp[:, :, slots < 0] = -1e6
    rp = np.arange(nb + 1) * nb
    ci = np.tile(np.arange(nb), nb).astype(np.int32)
    out = orc.attention(qp, kp, vp, rp, ci, N, Bk, 1 / sqrt(D), counts=counts)
    got = orc.permute_inv(np.nan_to_num(out), grid, tile, pad3d=True)
    ref = orc.dense_attention(q, k, v, 1 / sqrt(D))
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    assert orc.kept_flops(rp, ci, N, Bk, D, counts=counts) == 4 * N * N * D
