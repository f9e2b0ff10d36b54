"""The list-comparison rule of ``oracle.parity`` on crafted score rows: equal
lists pass, a swap between two blocks whose scores sit within 1e-4 of the
row's threshold is tolerated, and a swap far from it, a difference inside the
diagonal band, or a missing block in fixed mode fail."""
import numpy as np

from oracle import parity
from oracle import svsa_oracle as orc


def _csr(rows):
    rp = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int64)
    ci = np.concatenate([np.asarray(r, np.int32) for r in rows]) if rows else np.zeros(0, np.int32)
    return rp, ci


def _scores():
    # one head, nb = 6; row 0 carries two near-equal scores at the threshold
    s = np.array([[0.40, 0.30, 0.15, 0.149995, 0.00001, 0.000005],
                  [0.05, 0.60, 0.20, 0.10, 0.03, 0.02],
                  [0.10, 0.10, 0.50, 0.20, 0.05, 0.05],
                  [0.05, 0.05, 0.10, 0.60, 0.15, 0.05],
                  [0.02, 0.03, 0.05, 0.10, 0.70, 0.10],
                  [0.01, 0.01, 0.03, 0.05, 0.10, 0.80]])
    return s / s.sum(axis=1, keepdims=True)


def test_equal_lists_and_near_threshold_swap():
    S = _scores()[None, None]
    tp = np.array([0.8], np.float32)
    rp, ci = orc.block_mask(S, 1, top_p=tp)
    tol, bad = parity.mask_mismatch(S, 1, rp, ci, rp, ci, top_p=tp)
    assert tol == [] and bad == []
    rows = [list(ci[rp[r]: rp[r + 1]]) for r in range(6)]
    assert 2 in rows[0] and 3 not in rows[0]
    swapped = [sorted([j for j in rows[0] if j != 2] + [3])] + rows[1:]
    g_rp, g_ci = _csr(swapped)
    tol, bad = parity.mask_mismatch(S, 1, g_rp, g_ci, rp, ci, top_p=tp)
    assert tol == [0] and bad == []


def test_far_swap_band_difference_and_fixed_mode_fail():
    S = _scores()[None, None]
    tp = np.array([0.8], np.float32)
    rp, ci = orc.block_mask(S, 1, top_p=tp)
    rows = [list(ci[rp[r]: rp[r + 1]]) for r in range(6)]
    far = list(rows)
    far[1] = sorted([j for j in rows[1] if j != 2] + [5])       # 0.20 for 0.02
    g_rp, g_ci = _csr(far)
    assert parity.mask_mismatch(S, 1, g_rp, g_ci, rp, ci, top_p=tp) == ([], [1])
    band = list(rows)
    band[4] = [j for j in rows[4] if j != 4]                    # drops the diagonal
    g_rp, g_ci = _csr(band)
    assert parity.mask_mismatch(S, 1, g_rp, g_ci, rp, ci, top_p=tp) == ([], [4])
    kf = np.array([0.5], np.float32)
    rp, ci = orc.block_mask(S, 1, keep_frac=kf)
    rows = [list(ci[rp[r]: rp[r + 1]]) for r in range(6)]
    short = list(rows)
    short[5] = [j for j in rows[5] if j != 4]                   # 0.10, above tau 0.05
    g_rp, g_ci = _csr(short)
    tol, bad = parity.mask_mismatch(S, 1, g_rp, g_ci, rp, ci, keep_frac=kf)
    assert bad == [5]


def test_error_accumulator_matches_direct_formulas():
    rng = np.random.default_rng(3)
    ref = rng.standard_normal((10, 8))
    g32 = (ref + 1e-3 * rng.standard_normal(ref.shape)).astype(np.float32)
    acc = parity.ErrorAccumulator()
    acc.add(g32[:4], ref[:4], key=0)
    acc.add(g32[4:], ref[4:], key=1)
    d = g32.astype(np.float64) - ref
    assert acc.max_abs == np.abs(d).max() and acc.rows == 10
    assert np.isclose(acc.rel_l2, np.linalg.norm(d) / np.linalg.norm(ref), rtol=1e-12)
    per = acc.rel_l2_per_key()
    assert np.isclose(per[1], np.linalg.norm(d[4:]) / np.linalg.norm(ref[4:]), rtol=1e-12)
