"""Pins for the oracle's k-means (CPU only): exact 1-D k-means against brute
force over every assignment of tiny inputs, and Lloyd's textbook invariants."""

import itertools

import numpy as np

from oracle import kmeans


def _brute_1d(v, k):
    best = np.inf
    for lab in itertools.product(range(k), repeat=len(v)):
        lab = np.array(lab)
        if len(set(lab)) < k:
            continue
        sse = sum(np.sum((v[lab == c] - v[lab == c].mean()) ** 2) for c in range(k))
        best = min(best, sse)
    return best


def test_exact_1d_vs_brute_force():
    rng = np.random.default_rng(0)
    for trial in range(8):
        n, k = (7, 3) if trial % 2 else (6, 2)
        v = rng.standard_normal((1, n)) * rng.uniform(0.1, 3)
        centers, sse = kmeans.kmeans_1d_exact(v, k)
        assert abs(sse[0] - _brute_1d(v[0], k)) < 1e-9
        assert np.all(np.diff(centers[0]) >= 0)


def test_exact_1d_vectorised_rows_independent():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((5, 40))
    c_all, s_all = kmeans.kmeans_1d_exact(v, 6)
    for i in range(5):
        c1, s1 = kmeans.kmeans_1d_exact(v[i:i + 1], 6)
        assert np.allclose(c1[0], c_all[i]) and np.isclose(s1[0], s_all[i])


def test_exact_1d_recovers_separated_clusters():
    v = np.array([[0.0, 0.1, 0.2, 5.0, 5.1, 9.0, 9.2, 9.4]])
    centers, sse = kmeans.kmeans_1d_exact(v, 3)
    assert np.allclose(centers[0], [0.1, 5.05, 9.2])


def test_lloyd_objective_non_increasing_and_fixed_point():
    rng = np.random.default_rng(2)
    pts = np.concatenate([rng.standard_normal((200, 3)) + off for off in (0, 6, 12)])
    centers, assign, hist = kmeans.lloyd(pts, 5, 50, seed=3, return_history=True)
    assert all(b <= a + 1e-9 for a, b in zip(hist, hist[1:]))
    # at convergence: every point sits with its nearest center, centers are means
    assert np.array_equal(kmeans.assign_nearest(pts, centers), assign)
    for c in range(5):
        if np.any(assign == c):
            assert np.allclose(centers[c], pts[assign == c].mean(axis=0))


def test_lloyd_six_points_two_clusters_optimal():
    pts = np.array([[0, 0], [0, 1], [1, 0], [10, 10], [10, 11], [11, 10]], dtype=np.float64)
    best = min(
        kmeans.sse_of_assignment(pts, np.array([pts[np.array(l) == c].mean(0) for c in (0, 1)]), np.array(l))
        for l in itertools.product((0, 1), repeat=6) if 0 < sum(l) < 6)
    centers, assign = kmeans.lloyd(pts, 2, 20, seed=0)
    assert abs(kmeans.sse_of_assignment(pts, centers, assign) - best) < 1e-9
