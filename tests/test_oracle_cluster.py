"""Pins of the oracle's variable-size (cluster) blocks ([iCATS] Sec. 3.1,
4.1; [SVOO] QK co-clustering).  The pages describe the idea only; these pins
fix the reading against library routines and closed forms."""
import json
import os
import warnings

import numpy as np
import pytest

from oracle import svsa_oracle as orc


def _scipy_kmeans(x, c0, iters):
    from scipy.cluster.vq import kmeans2
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        return kmeans2(x, c0.copy(), iter=iters, minit="matrix", missing="warn")


def _data(seed, n=60, d=4, c=6):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d))
    c0 = x[rng.choice(n, c, replace=False)].copy()
    return x, c0


@pytest.mark.parametrize("seed,iters", [(0, 1), (1, 3), (2, 8)])
def test_kmeans_euclidean_equals_scipy(seed, iters):
    x, c0 = _data(seed)
    c0[-1] = 50.0                                   # one cluster stays empty
    c, sizes, lab = orc.kmeans(x, c0, iters)
    c_ref, lab_ref = _scipy_kmeans(x, c0, iters)
    assert np.array_equal(lab, lab_ref)
    np.testing.assert_allclose(c, c_ref, rtol=0, atol=1e-12)
    assert sizes[-1] == 0 and np.all(c[-1] == 50.0) and sizes.sum() == x.shape[0]


@pytest.mark.parametrize("seed", [3, 4])
def test_kmeans_metric_equals_scipy_after_cholesky(seed):
    """(x - c)^T G (x - c) = |(x - c) L|^2 for G = L L^T: k-means under G is
    Euclidean k-means of the rows x L, and means commute with L."""
    x, c0 = _data(seed)
    rng = np.random.default_rng(seed + 10)
    A = rng.standard_normal((4, 4))
    G = A @ A.T + 0.1 * np.eye(4)
    L = np.linalg.cholesky(G)
    c, _, lab = orc.kmeans(x, c0, 4, G)
    c_ref, lab_ref = _scipy_kmeans(x @ L, c0 @ L, 4)
    assert np.array_equal(lab, lab_ref)
    np.testing.assert_allclose(c @ L, c_ref, rtol=0, atol=1e-10)


def test_quad_distances_equal_squared_mahalanobis():
    from scipy.spatial.distance import cdist
    x, c0 = _data(5)
    rng = np.random.default_rng(6)
    A = rng.standard_normal((4, 4))
    G = A @ A.T + np.eye(4)
    np.testing.assert_allclose(orc.quad_distances(x, c0, G),
                               cdist(x, c0, "mahalanobis", VI=G) ** 2, rtol=1e-12)
    np.testing.assert_allclose(orc.quad_distances(x, c0), cdist(x, c0, "sqeuclidean"),
                               rtol=1e-12)


def test_kmeans_assign_ties_go_to_the_lowest_index():
    x = np.array([[0.0, 0.0], [1.0, 1.0]])
    c = np.array([[2.0, 2.0], [0.5, 0.5], [0.5, 0.5], [-0.5, -0.5]])
    assert orc.kmeans_assign(x, c).tolist() == [1, 1]


def test_cluster_metric_is_the_interaction_error():
    """With every key its own cluster, (q - mu)^T G (q - mu) equals the summed
    squared change of the logits sum_k ((q - mu) . k)^2, and G = K^T K."""
    rng = np.random.default_rng(7)
    K = rng.standard_normal((30, 5))
    G = orc.cluster_metric(K, np.ones(30))
    np.testing.assert_allclose(G, np.matmul(K.T, K), rtol=1e-12)
    q, mu = rng.standard_normal(5), rng.standard_normal(5)
    brute = sum(float(np.dot(q - mu, k)) ** 2 for k in K)
    assert abs(orc.quad_distances(q[None], mu[None], G)[0, 0] - brute) <= 1e-10 * brute
    # clusters of identical keys: size n_j times one copy
    G2 = orc.cluster_metric(K[:3], np.array([2, 1, 4]))
    np.testing.assert_allclose(G2, np.matmul(K[[0, 0, 1, 2, 2, 2, 2]].T, K[[0, 0, 1, 2, 2, 2, 2]]),
                               rtol=1e-12)


def test_cluster_means_closed_form():
    x = np.arange(24, dtype=np.float64).reshape(1, 1, 6, 4)
    lab = np.array([[[1, 0, 1, 1, 0, 3]]])
    m, n = orc.cluster_means(x, lab, 4)
    assert n[0, 0].tolist() == [2, 3, 0, 1]
    np.testing.assert_array_equal(m[0, 0, 0], (x[0, 0, 1] + x[0, 0, 4]) / 2)
    np.testing.assert_array_equal(m[0, 0, 1], (x[0, 0, 0] + x[0, 0, 2] + x[0, 0, 3]) / 3)
    assert np.all(np.isnan(m[0, 0, 2]))


def test_cluster_layout_hand_worked(golden_dir):
    with open(os.path.join(golden_dir, "cluster_layout.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        start, slot, token = orc.cluster_layout(np.array(c["labels"]), c["clusters"], c["align"])
        assert start.tolist() == c["start"]
        assert slot.tolist() == c["slot"]
        assert token.tolist() == c["token"]


def test_cluster_permute_round_trip_and_zero_padding():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((37, 3))
    lab = rng.integers(0, 5, 37)
    start, slot, token = orc.cluster_layout(lab, 5, 8)
    xp = orc.cluster_permute(x, token)
    assert np.all(xp[token < 0] == 0) and xp.shape[0] == start[-1]
    assert np.array_equal(orc.cluster_unpermute(xp, slot), x)


def test_cluster_scores_weight_by_size():
    """Identical key centroids: the scores are the size fractions n_j / N
    (empty clusters 0), whatever the query."""
    rng = np.random.default_rng(9)
    qbar = rng.standard_normal((3, 4))
    kbar = np.tile(rng.standard_normal(4), (4, 1))
    S = orc.cluster_scores(qbar, kbar, np.array([5, 3, 0, 2]), 0.7)
    np.testing.assert_allclose(S, np.tile([0.5, 0.3, 0.0, 0.2], (3, 1)), rtol=1e-14, atol=0)
    # one channel, two equal-size clusters: logistic in the logit difference
    S = orc.cluster_scores(np.array([[2.0]]), np.array([[1.0], [-1.0]]), np.array([4, 4]), 0.5)
    assert abs(S[0, 0] - 1 / (1 + np.exp(-2.0))) < 1e-15


def test_cluster_scores_ignore_undefined_empty_centroids():
    """Empty key clusters score 0 even when their centroid is undefined (the
    NaN mean of no tokens), and leave the other scores as without them."""
    rng = np.random.default_rng(13)
    qbar, kbar = rng.standard_normal((2, 3)), rng.standard_normal((4, 3))
    kb = kbar.copy()
    kb[1] = np.nan
    S = orc.cluster_scores(qbar, kb, np.array([3, 0, 2, 5]), 0.4)
    ref = orc.cluster_scores(qbar, kbar[[0, 2, 3]], np.array([3, 2, 5]), 0.4)
    assert np.all(S[:, 1] == 0.0) and np.all(np.isfinite(S))
    np.testing.assert_allclose(S[:, [0, 2, 3]], ref, rtol=1e-14)


def test_cluster_mask_top_p_on_size_fractions():
    S = np.tile([0.5, 0.3, 0.0, 0.2], (1, 1, 2, 1))
    rp, ci = orc.cluster_mask(S, top_p=np.array([0.7], np.float32))
    assert rp.tolist() == [0, 2, 4] and ci.tolist() == [0, 1, 0, 1]
    rp, ci = orc.cluster_mask(S, keep_frac=np.array([0.75], np.float32))
    assert ci[: rp[1]].tolist() == [0, 1, 3]


def test_cluster_attention_all_kept_equals_dense_sdpa():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(10)
    q, k, v = (rng.standard_normal((40, 8)) for _ in range(3))
    qlab, klab = rng.integers(0, 4, 40), rng.integers(0, 6, 40)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a)[None] for a in (q, k, v)), scale=0.3)[0].numpy()
    for i in range(4):
        toks, out = orc.cluster_attention_rows(q, k, v, qlab, klab, i, np.arange(6), 0.3)
        np.testing.assert_allclose(out, ref[toks], rtol=1e-12, atol=1e-12)
    # one kept key cluster: plain softmax attention over exactly its members
    toks, out = orc.cluster_attention_rows(q, k, v, qlab, klab, 2, [1], 0.3)
    km = klab == 1
    ref2 = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[toks])[None], torch.from_numpy(k[km])[None],
        torch.from_numpy(v[km])[None], scale=0.3)[0].numpy()
    np.testing.assert_allclose(out, ref2, rtol=1e-12, atol=1e-12)
