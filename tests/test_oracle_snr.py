"""Pins of the oracle's SNR-guided top-p schedule ([iCATS] Sec. 4.2, App. A).

The pages fix the schedule's shape and parameters, not its formula, so these
pins fix the reading (hand-worked values, limits, monotonicity, the symmetry
of the sigmoid) rather than a published number: parity unpinned against the
pages' own formula."""
import json
import os

import numpy as np

from oracle import svsa_oracle as orc


def _flow_sigmas(steps, shift):
    t = 1.0 - np.arange(steps) / steps
    return shift * t / (1.0 + (shift - 1.0) * t)


def test_snr_hand_worked_schedules(golden_dir):
    with open(os.path.join(golden_dir, "snr_schedule.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got = orc.snr_top_p(c["sigmas"], c["first_sparse"], c["p_min"], c["tau"])
        np.testing.assert_allclose(got, c["top_p"], rtol=0, atol=1e-12, err_msg=c["name"])


def test_snr_shape_over_a_shifted_flow_schedule():
    """Dense warmup, tau at the first sparse step, pmin at the last, never
    rising, and flatter at both ends than in the middle (the shape the pages
    describe)."""
    s = _flow_sigmas(50, 5.0)
    p = orc.snr_top_p(s, 10, 0.7, 0.999)
    assert np.all(p[:10] == 1.0)
    assert p[10] == 0.999 and abs(p[-1] - 0.7) < 1e-15
    d = -np.diff(p[10:])
    assert np.all(d >= -1e-15)
    assert d[:3].mean() < d.max() and d[-3:].mean() < d.max()


def test_snr_sigmoid_symmetry():
    """w(s) + w(1 - s) = 1: a schedule and its mirror give top-p values that
    mirror about the mid value (tau + pmin) / 2."""
    s = np.array([0.9, 0.7, 0.55, 0.3, 0.1])
    p = orc.snr_top_p(s, 0, 0.6, 1.0)
    q = orc.snr_top_p(1.0 - s[::-1], 0, 0.6, 1.0)
    np.testing.assert_allclose(p + q[::-1], 1.6, atol=1e-12)


def test_snr_constant_noise_level_keeps_tau():
    p = orc.snr_top_p([0.4, 0.4, 0.4], 1, 0.7, 0.98)
    assert p.tolist() == [1.0, 0.98, 0.98]
