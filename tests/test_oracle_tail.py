"""Pins of the oracle's tail merging ([iCATS] Sec. 4.3, App. E.1 reading)."""
import json
import os

import numpy as np

from oracle import svsa_oracle as orc


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "tail_merge.json")) as f:
        g = json.load(f)
    K = np.zeros((len(g["kept"]), g["nk"]), bool)
    for i, r in enumerate(g["kept"]):
        K[i, r] = True
    return g, K


def test_tail_merge_hand_worked(golden_dir):
    g, K = _golden(golden_dir)
    lab, R, sizes = orc.tail_merge(g["labels"], K, g["block"])
    assert lab.tolist() == g["out_labels"]
    assert [np.nonzero(r)[0].tolist() for r in R] == g["out_kept"]
    assert sizes.tolist() == g["out_sizes"]


def _random_case(seed, C=12, nk=9, N=200, block=8):
    rng = np.random.default_rng(seed)
    K = rng.random((C, nk)) < 0.4
    K[3] = K[7]                     # identical kept sets
    K[10] = K[1]
    lab = rng.integers(0, C, size=N)
    lab[lab == 5] = 4               # an empty cluster
    return lab, K, block


def test_tail_merge_invariants():
    for seed in range(6):
        lab0, K0, b = _random_case(seed)
        lab, R, sizes = orc.tail_merge(lab0, K0, b)
        assert sizes.sum() == lab0.size and np.array_equal(np.bincount(lab, minlength=12), sizes)
        # the attention pattern of every token only grows
        assert np.all(~K0[lab0] | R[lab])
        # padded blocks never increase
        before = np.sum(-(-np.bincount(lab0, minlength=12) // b))
        assert np.sum(-(-sizes // b)) <= before


def test_tail_merge_without_rounds_merges_identical_sets_only():
    for seed in range(4):
        lab0, K0, b = _random_case(seed)
        lab, R, sizes = orc.tail_merge(lab0, K0, b, rounds=0)
        used = np.unique(lab0)
        distinct = {K0[i].tobytes() for i in used}
        assert np.count_nonzero(sizes) == len(distinct)
        assert np.array_equal(R, K0)
        # a token moves only to the lowest cluster with its kept set
        for t in range(lab0.size):
            same = [j for j in used if np.array_equal(K0[j], K0[lab0[t]])]
            assert lab[t] == min(same)


def test_tail_merge_equal_tails_higher_index_donates():
    # two clusters of 6 tokens, block 4: tails 2 + 2 fit; cluster 1 donates
    lab = np.array([0, 1] * 6)
    K = np.array([[1, 0, 1], [1, 1, 0]], bool)
    out, R, sizes = orc.tail_merge(lab, K, 4)
    assert sizes.tolist() == [8, 4]
    assert out.tolist() == [0, 1, 0, 1, 0, 1, 0, 1, 0, 0, 0, 0]
    assert R[0].tolist() == [True, True, True] and R[1].tolist() == [True, True, False]
