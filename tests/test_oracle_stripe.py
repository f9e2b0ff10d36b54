"""Pins of the oracle's stripe masks ([PSA] Alg. 1 at tile granularity)."""
import json
import os

import numpy as np

from oracle import svsa_oracle as orc


def _csr_rows(rp, ci):
    return [list(ci[rp[r]:rp[r + 1]]) for r in range(len(rp) - 1)]


def test_stripe_hand_worked_examples(golden_dir=None):
    golden_dir = golden_dir or os.path.join(os.path.dirname(__file__), "golden")
    with open(os.path.join(golden_dir, "psa_alg1_examples.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        rp, ci = orc.stripe_mask(tuple(c["grid"]), tuple(c["tile"]), [c["params"]], c["band"])
        assert _csr_rows(rp, ci) == c["rows"], c["name"]


def test_stripe_svg_special_case_is_a_plain_window():
    # [PSA] Sec. 3.2: SVG is M(Tw, 0, inf, Sw, 0, inf): a window |dt| < Tw, |ds| < Sw
    rng = np.random.default_rng(3)
    ti, si, tj, sj = (rng.integers(0, 9, 400) for _ in range(4))
    for Tw, Sw in ((1, 1), (2, 3), (4, 1), (3, 5)):
        got = orc.psa_attends(ti, si, tj, sj, (Tw, 0, 0, Sw, 0, 0))
        want = (np.abs(tj - ti) < Tw) & (np.abs(sj - si) < Sw)
        assert np.array_equal(got, want)


def test_stripe_stride_repeats_the_band():
    # a finite stride repeats the band every Ts frames (Ss positions) past the offset
    for Tw, To, Ts in ((1, 0, 2), (2, 1, 3), (1, -2, 3)):
        d = np.arange(To, To + 12)
        a = orc.psa_attends(0, 0, d, 0, (Tw, To, Ts, 1, 0, 0))
        b = orc.psa_attends(0, 0, d + Ts, 0, (Tw, To, Ts, 1, 0, 0))
        assert np.array_equal(a, b)
        assert a[0] and a.sum() == Tw * (len(d) // Ts) + min(Tw, len(d) % Ts)
    for Sw, So, Ss in ((1, 1, 5), (2, 0, 6)):
        d = np.arange(So, So + 15)
        a = orc.psa_attends(0, 0, 0, d, (1, 0, 0, Sw, So, Ss))
        assert np.array_equal(a, orc.psa_attends(0, 0, 0, d + Ss, (1, 0, 0, Sw, So, Ss)))


def test_stripe_offset_direction():
    # To = +1: the kept key frame is one frame after the query frame
    assert orc.psa_attends(2, 0, 3, 0, (1, 1, 0, 1, 0, 0))
    assert not orc.psa_attends(2, 0, 1, 0, (1, 1, 0, 1, 0, 0))
    assert orc.psa_attends(0, 5, 0, 3, (1, 0, 0, 1, -2, 0))
    assert not orc.psa_attends(0, 5, 0, 7, (1, 0, 0, 1, -2, 0))


def test_stripe_limits_and_monotone():
    grid, tile = (5, 6, 8), (2, 4, 4)   # partial tiles: blocks mix tiles
    tiles = orc.block_tiles(grid, tile)
    nb = len(tiles)
    nT, nH, nW = 3, 2, 2
    rp, ci = orc.stripe_mask(grid, tile, [[nT, 0, 0, nH * nW, 0, 0]], 0)
    assert all(len(r) == nb for r in _csr_rows(rp, ci))           # full window
    small = _csr_rows(*orc.stripe_mask(grid, tile, [[1, 0, 2, 1, 1, 3]], 0))
    big = _csr_rows(*orc.stripe_mask(grid, tile, [[2, 0, 2, 2, 1, 3]], 0))
    assert all(set(a) <= set(b) for a, b in zip(small, big))
    banded = _csr_rows(*orc.stripe_mask(grid, tile, [[1, 0, 2, 1, 1, 3]], 2))
    for i, (a, b) in enumerate(zip(small, banded)):
        assert set(b) == set(a) | {j for j in (i - 1, i, i + 1) if 0 <= j < nb}


def test_stripe_blocks_use_every_token_tile():
    # a block keeps a key block iff some token pair's tiles attend (token-level
    # brute force over the tile of every token, no de-duplication)
    grid, tile = (3, 5, 6), (2, 2, 4)
    T, H, W = grid
    tt, th, tw = tile
    nW = -(-W // tw)
    pi = orc.tile_order(grid, tile)
    t, rem = np.divmod(pi, H * W)
    h, w = np.divmod(rem, W)
    tp, sp = t // tt, (h // th) * nW + w // tw
    Bk = tt * th * tw
    N = T * H * W
    nb = -(-N // Bk)
    params = (1, 1, 0, 2, -1, 3)
    rows = _csr_rows(*orc.stripe_mask(grid, tile, [params], 0))
    for i in range(nb):
        qi = np.arange(i * Bk, min((i + 1) * Bk, N))
        want = []
        for j in range(nb):
            kj = np.arange(j * Bk, min((j + 1) * Bk, N))
            hit = False
            for q in qi:
                for k in kj:
                    if orc.psa_attends(tp[q], sp[q], tp[k], sp[k], params):
                        hit = True
                        break
                if hit:
                    break
            if hit:
                want.append(j)
        assert rows[i] == want
