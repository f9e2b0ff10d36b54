"""Pins of the oracle's block scores (stage 3a) and top-p / fixed selection (3b)."""
from itertools import combinations
from math import ceil, fsum, exp, sqrt

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

from oracle import svsa_oracle as orc
from svsa_synth import make_inputs


def _tiny_scores():
    inp = make_inputs("tiny")
    cfg = inp.cfg
    qp = orc.permute_fwd(inp.q32, cfg.grid, cfg.tile)
    kp = orc.permute_fwd(inp.k32, cfg.grid, cfg.tile)
    qb = orc.pool(qp, cfg.N, cfg.Bk)
    kb = orc.pool(kp, cfg.N, cfg.Bk)
    return cfg, qb, kb, orc.block_scores(qb, kb, 1 / sqrt(cfg.head_dim))


def test_scores_match_library_softmax_of_brute_force_logits():
    cfg, qb, kb, S = _tiny_scores()
    nb, D = cfg.nb, cfg.head_dim
    L = np.array([[fsum(qb[0, 0, i, d] * kb[0, 0, j, d] for d in range(D)) / sqrt(D)
                   for j in range(nb)] for i in range(nb)])
    np.testing.assert_allclose(S[0, 0], sp_softmax(L, axis=1), rtol=1e-12, atol=0)
    np.testing.assert_allclose(S.sum(-1), 1.0, atol=1e-12)


def test_scores_closed_form_one_channel():
    # Qbar_i = a_i e_0, Kbar_j = c_j e_0  =>  S_ij = exp(a_i c_j / sqrt D) / sum_j'
    D = 16
    a = np.array([1.0, -2.0, 0.5])
    c = np.array([0.3, 1.1, -0.7, 2.0])
    qb = np.zeros((1, 1, 3, D)); qb[0, 0, :, 0] = a
    kb = np.zeros((1, 1, 4, D)); kb[0, 0, :, 0] = c
    S = orc.block_scores(qb, kb, 1 / sqrt(D))
    for i in range(3):
        e = [exp(a[i] * cj / 4.0) for cj in c]
        z = fsum(e)
        np.testing.assert_allclose(S[0, 0, i], [x / z for x in e], rtol=1e-14)
    # rows depend on Qbar_i, not on Kbar_i (guards against a transposed operand)
    assert not np.allclose(S[0, 0, 0], S[0, 0, 1])


def _brute_force_topp(s, p):
    """min cardinality of a subset reaching mass p; max mass at that size."""
    nb = s.size
    for k in range(1, nb + 1):
        best = max(fsum(s[list(c)]) for c in combinations(range(nb), k))
        if best >= p:
            return k, best
    return nb, fsum(s)


@pytest.mark.parametrize("p", [0.3, 0.5, 0.9, 0.99])
def test_topp_brute_force_on_tiny(p):
    cfg, _, _, S = _tiny_scores()
    nb = cfg.nb
    for i in range(nb):
        s = S[0, 0, i]
        kstar, best = _brute_force_topp(s, p)
        kept = orc.select_row(s, i, band=0, top_p=np.float32(p))   # band 0: top-p only
        p32 = float(np.float32(p))
        if abs(best - p32) > 1e-12:   # away from an exact tie with p
            assert kept.size == kstar
            assert abs(fsum(s[kept]) - best) < 1e-12
        # with the band added the diagonal is always present
        kept_b = orc.select_row(s, i, band=1, top_p=np.float32(p))
        assert i in kept_b and set(kept) <= set(kept_b.tolist())
        assert np.all(np.diff(kept_b) > 0)


def test_topp_monotone_and_limits():
    cfg, _, _, S = _tiny_scores()
    nb = cfg.nb
    for i in range(nb):
        s = S[0, 0, i]
        prev = set()
        for p in (1e-6, 0.2, 0.5, 0.8, 0.9, 0.999, 1.0):
            cur = set(orc.select_row(s, i, band=1, top_p=np.float32(p)).tolist())
            assert prev <= cur
            prev = cur
        assert prev == set(range(nb))                                  # p = 1 keeps all
        tiny_p = set(orc.select_row(s, i, band=1, top_p=np.float32(1e-6)).tolist())
        assert tiny_p == {int(np.argmax(s)), i}                        # p -> 0+: argmax + band


def test_topp_tie_break_lower_index():
    s = np.array([0.1, 0.25, 0.25, 0.25, 0.15])
    # top-2 by score: ties among 1,2,3 go to the lower indices 1 and 2
    assert orc.select_row(s, 4, band=0, top_p=np.float32(0.5)).tolist() == [1, 2]
    assert orc.select_row(s, 0, band=1, top_p=np.float32(0.5)).tolist() == [0, 1, 2]


def test_band_width():
    s = np.zeros(10); s[0] = 1.0
    assert orc.select_row(s, 5, band=3, top_p=np.float32(0.5)).tolist() == [0, 3, 4, 5, 6, 7]
    assert orc.select_row(s, 9, band=2, top_p=np.float32(0.5)).tolist() == [0, 8, 9]


def test_fixed_fraction_mode():
    cfg, _, _, S = _tiny_scores()
    nb = cfg.nb
    for f in (0.1, 0.3, 0.5, 1.0):
        k = ceil(float(np.float32(f)) * nb)
        for i in range(nb):
            s = S[0, 0, i]
            kept = orc.select_row(s, i, band=0, keep_frac=np.float32(f))
            assert kept.size == k
            top = np.argsort(-s, kind="stable")[:k]
            assert set(kept.tolist()) == set(top.tolist())
            assert s[kept].min() >= np.delete(s, kept).max(initial=-1)


def test_block_mask_csr_layout():
    cfg, _, _, S = _tiny_scores()
    rp, ci = orc.block_mask(S, band=1, top_p=np.array([0.9], np.float32))
    assert rp.shape == (cfg.nb + 1,) and rp[0] == 0 and rp[-1] == ci.size
    for i in range(cfg.nb):
        row = ci[rp[i]: rp[i + 1]]
        assert row.tolist() == orc.select_row(S[0, 0, i], i, 1, top_p=np.float32(0.9)).tolist()


def test_topp_reaching_p_exactly_is_inclusive():
    # 0.5 + 0.25 reaches 0.75 exactly (all values exact in binary): two blocks suffice
    s = np.array([0.5, 0.25, 0.25])
    assert orc.select_row(s, 0, band=0, top_p=np.float32(0.75)).tolist() == [0, 1]
    assert orc.select_row(s, 0, band=0, top_p=np.float32(0.7500001)).tolist() == [0, 1, 2]


def test_fixed_fraction_count_uses_the_float32_fraction():
    # k = ceil(f * nb) with f the float32 value of the fraction, widened
    # exactly: float32(0.3) = 0.300000011920928955..., so 10 blocks keep 4;
    # 0.25 is exact in binary, so 8 blocks keep 2; a tiny fraction still
    # keeps the top block, and the count never exceeds nb.
    assert float(np.float32(0.3)) > 0.3
    s = np.linspace(1.0, 2.0, 10)[::-1] / fsum(np.linspace(1.0, 2.0, 10))
    assert orc.select_row(s, 9, band=0, keep_frac=np.float32(0.3)).tolist() == [0, 1, 2, 3]
    s8 = np.array([0.05, 0.3, 0.1, 0.2, 0.05, 0.1, 0.15, 0.05])
    assert orc.select_row(s8, 0, band=0, keep_frac=np.float32(0.25)).tolist() == [1, 3]
    assert orc.select_row(s8, 0, band=0, keep_frac=np.float32(1e-6)).tolist() == [1]
    assert orc.select_row(s8, 0, band=0, keep_frac=np.float32(1.0)).tolist() == list(range(8))
    # the band is added after the count and does not count toward it
    assert orc.select_row(s8, 5, band=2, keep_frac=np.float32(0.25)).tolist() == [1, 3, 4, 5, 6]
    # equal scores at the cut go to the lower key index, as in top-p
    s4 = np.array([0.1, 0.3, 0.3, 0.3])
    assert orc.select_row(s4, 0, band=0, keep_frac=np.float32(0.5)).tolist() == [1, 2]
