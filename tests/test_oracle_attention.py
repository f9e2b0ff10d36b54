"""Pins of the oracle's block-sparse attention (stage 4) and FLOP accounting."""
import json
import os
from math import sqrt

import numpy as np
import pytest
import torch
from scipy.special import softmax as sp_softmax

from oracle import svsa_oracle as orc
from svsa_synth import make_inputs


def _all_blocks_csr(rows, nb):
    rp = np.arange(rows + 1, dtype=np.int64) * nb
    ci = np.tile(np.arange(nb, dtype=np.int32), rows)
    return rp, ci


def _torch_sdpa(q, k, v, scale):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=scale).numpy()


@pytest.mark.parametrize("grid,tile", [((4, 8, 8), (2, 4, 4)), ((3, 5, 6), (2, 2, 4))])
def test_all_blocks_kept_equals_dense_sdpa(grid, tile):
    rng = np.random.default_rng(3)
    B, Hh, D = 1, 2, 32
    N = int(np.prod(grid)); Bk = int(np.prod(tile)); nb = orc.num_blocks(N, Bk)
    q, k, v = (rng.standard_normal((B, Hh, N, D)).astype(np.float32) for _ in range(3))
    scale = 1 / sqrt(D)
    qp, kp, vp = (orc.permute_fwd(x, grid, tile) for x in (q, k, v))
    rp, ci = _all_blocks_csr(B * Hh * nb, nb)
    out = orc.permute_inv(orc.attention(qp, kp, vp, rp, ci, N, Bk, scale), grid, tile)
    ref = _torch_sdpa(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), scale)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(orc.dense_attention(q, k, v, scale), ref, rtol=0, atol=1e-12)


def test_sparse_rows_are_convex_combinations_of_kept_values():
    inp = make_inputs("small", heads=[0, 3])
    cfg = inp.cfg
    N, Bk, nb, D = cfg.N, cfg.Bk, cfg.nb, cfg.head_dim
    qp, kp, vp = (orc.permute_fwd(x, cfg.grid, cfg.tile) for x in (inp.q, inp.k, inp.v))
    S = orc.block_scores(orc.pool(qp, N, Bk), orc.pool(kp, N, Bk), 1 / sqrt(D))
    rp, ci = orc.block_mask(S, 1, top_p=np.full(2, 0.9, np.float32))
    out = orc.attention(qp, kp, vp, rp, ci, N, Bk, 1 / sqrt(D))
    for h in range(2):
        for i in range(nb):
            r = h * nb + i
            cols = ci[rp[r]: rp[r + 1]]
            keys = np.concatenate([np.arange(j * Bk, (j + 1) * Bk) for j in cols])
            vk = vp[0, h, keys]
            o = out[0, h, i * Bk:(i + 1) * Bk]
            assert np.all(o >= vk.min(axis=0) - 1e-12) and np.all(o <= vk.max(axis=0) + 1e-12)


def test_constant_values_give_constant_output():
    grid, tile = (3, 5, 6), (2, 2, 4)
    N, Bk, D = 90, 16, 8
    nb = orc.num_blocks(N, Bk)
    rng = np.random.default_rng(0)
    q, k = (rng.standard_normal((1, 1, N, D)) for _ in range(2))
    v = np.full((1, 1, N, D), -1.75)
    qp, kp, vp = (orc.permute_fwd(x, grid, tile) for x in (q, k, v))
    rp = np.array([0, 1, 3, 4, 6, 7, 9]); ci = np.array([0, 0, 1, 2, 1, 3, 4, 2, 5], np.int32)
    out = orc.attention(qp, kp, vp, rp, ci, N, Bk, 0.3)
    valid = ~np.isnan(out)
    assert np.abs(out[valid] + 1.75).max() < 1e-14


def test_single_kept_block_is_local_attention():
    grid, tile = (3, 5, 6), (2, 2, 4)
    N, Bk, D = 90, 16, 8
    nb = orc.num_blocks(N, Bk)
    rng = np.random.default_rng(2)
    qp, kp, vp = (orc.permute_fwd(rng.standard_normal((1, 1, N, D)), grid, tile) for _ in range(3))
    rp = np.arange(nb + 1); ci = np.arange(nb, dtype=np.int32)   # diagonal only
    out = orc.attention(qp, kp, vp, rp, ci, N, Bk, 0.25)
    for i in range(nb):
        lo, hi = i * Bk, min((i + 1) * Bk, N)
        w = sp_softmax(qp[0, 0, lo:hi] @ kp[0, 0, lo:hi].T * 0.25, axis=1)
        np.testing.assert_allclose(out[0, 0, lo:hi], w @ vp[0, 0, lo:hi], atol=1e-13)
    # the tail block (10 valid keys) never sees padded keys
    assert np.all(np.isnan(out[0, 0, N:]))


def test_padded_keys_are_excluded():
    # Two blocks; padded tail rows of K are zero, so including them would pull
    # the softmax weights toward exp(0).  Compare with explicit valid-key attention.
    grid, tile = (1, 1, 20), (1, 1, 16)
    N, Bk, D = 20, 16, 4
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((1, 1, N, D)) for _ in range(3))
    qp, kp, vp = (orc.permute_fwd(x, grid, tile) for x in (q, k, v))
    rp = np.array([0, 2, 4]); ci = np.array([0, 1, 0, 1], np.int32)
    out = orc.attention(qp, kp, vp, rp, ci, N, Bk, 0.5)
    ref = orc.dense_attention(q, k, v, 0.5)
    np.testing.assert_allclose(out[0, 0, :N], ref[0, 0], atol=1e-13)


def test_kept_flops_reproduce_psa_table2_dense(golden_dir):
    rows = json.load(open(os.path.join(golden_dir, "psa_table2_dense.json")))["rows"]
    for r in rows:
        N = int(np.prod(r["grid"]))
        Bk = 64
        nb = orc.num_blocks(N, Bk)
        rp, ci = _all_blocks_csr(nb, nb)             # one head, every block kept
        f = orc.kept_flops(rp, ci, N, Bk, r["head_dim"]) * r["heads"]
        assert round(f / 1e12, 2) == r["tflop"], (r["model"], f / 1e12)


def test_kept_flops_counts_valid_tokens_only():
    N, Bk, D = 90, 16, 8
    rp = np.array([0, 1, 2, 3, 4, 5, 7]); ci = np.array([0, 1, 2, 3, 4, 0, 5], np.int32)
    # rows 0..4: 16*16 each; row 5 (tail, 10 valid): 10*16 + 10*10
    assert orc.kept_flops(rp, ci, N, Bk, D) == 4 * D * (5 * 256 + 160 + 100)


def test_sparse_row_closed_form_two_kept_blocks_with_a_tail():
    # Three blocks of two slots, N = 5 (block 2 holds one valid token and a
    # padding slot).  Query block 1 keeps blocks 0 and 2; keys are equal within
    # block 0, so with x_j = scale * q . k_j the weight of block 0 is the
    # logistic sigma(x_0 - x_2 + ln 2) (two keys against one) and the output is
    # that mix of block 0's mean value and block 2's one value.  Block 1 and the
    # padding slot carry huge keys and values: any leak shows at once.
    N, Bk, D, scale = 5, 2, 2, 0.7
    qp = np.zeros((1, 1, 6, D)); kp = np.zeros_like(qp); vp = np.zeros_like(qp)
    qp[0, 0, 2] = [1.0, 0.0]; qp[0, 0, 3] = [0.0, 1.0]           # query block 1
    kp[0, 0, 0:2] = [0.4, -1.2]; vp[0, 0, 0] = [1.0, 0.0]; vp[0, 0, 1] = [3.0, 0.0]
    kp[0, 0, 2:4] = 100.0; vp[0, 0, 2:4] = 1e3                     # block 1: not kept
    kp[0, 0, 4] = [-0.3, 0.9]; vp[0, 0, 4] = [0.0, 5.0]           # block 2, valid
    kp[0, 0, 5] = 50.0; vp[0, 0, 5] = 1e3                          # block 2, padding
    for cols in ([0, 2], [2, 0]):
        out = orc.attention_rows(qp, kp, vp, 0, 0, 1, cols, N, Bk, scale)
        for r, q in enumerate(([1.0, 0.0], [0.0, 1.0])):
            x0 = scale * float(np.dot(q, [0.4, -1.2]))
            x2 = scale * float(np.dot(q, [-0.3, 0.9]))
            w0 = 1.0 / (1.0 + np.exp(-(x0 - x2 + np.log(2.0))))
            np.testing.assert_allclose(out[r], [2.0 * w0, 5.0 * (1.0 - w0)], rtol=1e-13)
