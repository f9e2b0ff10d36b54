"""Pins of the oracle's tile order / permutation (stage 1) and pooling (stage 2)."""
import os

import numpy as np
import pytest

from oracle import svsa_oracle as orc
from svsa_synth import make_inputs


def _read_golden(path):
    vals = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = line.split("=")
        vals[k.strip()] = [int(x) for x in v.split()]
    return vals


def test_tile_order_worked_example(golden_dir):
    g = _read_golden(os.path.join(golden_dir, "c1_tile_order.txt"))
    pi = orc.tile_order((4, 8, 8), (2, 4, 4))
    assert pi[:32].tolist() == g["pi[0:32]"]
    assert pi[32:40].tolist() == g["pi[32:40]"]
    assert pi[::32].tolist() == g["block_start"]


@pytest.mark.parametrize("grid,tile", [((4, 8, 8), (2, 4, 4)), ((8, 16, 16), (4, 4, 4)),
                                       ((6, 9, 12), (3, 3, 4))])
def test_tile_order_equals_reshape_when_tiles_divide(grid, tile):
    # library route: reshape (nT,tt,nH,th,nW,tw) -> transpose -> flatten
    T, H, W = grid
    tt, th, tw = tile
    nat = np.arange(T * H * W).reshape(T // tt, tt, H // th, th, W // tw, tw)
    ref = nat.transpose(0, 2, 4, 1, 3, 5).ravel()
    assert np.array_equal(orc.tile_order(grid, tile), ref)


def _tile_order_loops(grid, tile):
    """Hand-written nested loops over tiles (partial edge tiles in place)."""
    T, H, W = grid
    tt, th, tw = tile
    out = []
    for a in range(0, T, tt):
        for b in range(0, H, th):
            for c in range(0, W, tw):
                for t in range(a, min(a + tt, T)):
                    for h in range(b, min(b + th, H)):
                        for w in range(c, min(c + tw, W)):
                            out.append((t * H + h) * W + w)
    return np.array(out)


@pytest.mark.parametrize("grid,tile", [((3, 5, 6), (2, 2, 4)), ((21, 30, 52), (4, 4, 4)),
                                       ((5, 7, 3), (4, 4, 4)), ((1, 1, 1), (2, 2, 2))])
def test_tile_order_partial_tiles_brute_force(grid, tile):
    pi = orc.tile_order(grid, tile)
    assert np.array_equal(pi, _tile_order_loops(grid, tile))
    assert np.array_equal(np.sort(pi), np.arange(np.prod(grid)))  # bijection


def test_permute_round_trip_bit_exact():
    rng = np.random.default_rng(5)
    grid, tile = (3, 5, 6), (2, 2, 4)
    N, Bk = 90, 16
    x = rng.integers(0, 2 ** 16, size=(2, 3, N, 8), dtype=np.uint16)
    x &= np.uint16(0x7F7F)  # keep bf16 patterns finite (exponent != 0xFF)
    xp = orc.permute_fwd(x, grid, tile)
    nb = orc.num_blocks(N, Bk)
    assert xp.shape == (2, 3, nb * Bk, 8)
    assert np.all(xp[:, :, N:] == 0)                      # zero-filled tail
    back = orc.permute_inv(xp, grid, tile)
    assert np.array_equal(back, orc.widen(x))


def test_permute_moves_rows_to_the_right_place():
    grid, tile = (3, 5, 6), (2, 2, 4)
    N = 90
    x = np.arange(N, dtype=np.float32).reshape(1, 1, N, 1).repeat(2, axis=3)
    xp = orc.permute_fwd(x, grid, tile)
    pi = _tile_order_loops(grid, tile)
    assert np.array_equal(xp[0, 0, :N, 0], pi.astype(np.float64))


def test_pool_equals_reshape_mean_when_tiles_divide():
    inp = make_inputs("small")
    grid, tile = inp.cfg.grid, inp.cfg.tile
    T, H, W = grid
    tt, th, tw = tile
    qf = orc.widen(inp.q)
    qp = orc.permute_fwd(inp.q, grid, tile)
    got = orc.pool(qp, inp.cfg.N, inp.cfg.Bk)
    B, Hh, N, D = qf.shape
    blocks = qf.reshape(B, Hh, T // tt, tt, H // th, th, W // tw, tw, D)
    ref = blocks.mean(axis=(3, 5, 7)).reshape(B, Hh, -1, D)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def test_pool_tail_uses_valid_count_and_constant_stays_constant():
    grid, tile = (3, 5, 6), (2, 2, 4)
    N, Bk = 90, 16
    x = np.full((1, 2, N, 4), 2.5, dtype=np.float32)
    xp = orc.permute_fwd(x, grid, tile)
    bars = orc.pool(xp, N, Bk)
    assert np.all(bars == 2.5)          # includes the tail block with 10 valid rows
    assert orc.block_valid_counts(N, Bk).tolist() == [16] * 5 + [10]


def test_pool_linearity():
    rng = np.random.default_rng(1)
    N, Bk = 90, 16
    grid, tile = (3, 5, 6), (2, 2, 4)
    a = rng.standard_normal((1, 1, N, 8))
    b = rng.standard_normal((1, 1, N, 8))
    pa = orc.pool(orc.permute_fwd(a, grid, tile), N, Bk)
    pb = orc.pool(orc.permute_fwd(b, grid, tile), N, Bk)
    pab = orc.pool(orc.permute_fwd(3 * a - b, grid, tile), N, Bk)
    np.testing.assert_allclose(pab, 3 * pa - pb, atol=1e-13)
