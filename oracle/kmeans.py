"""k-means used to learn the shared patterns (oracle; test infrastructure only).

The pages: each tensor has 64 patterns, each a list of 15 sorted centroids
fixed after offline learning (Ecco review, "What carries the argument"),
learned with k-means on calibration data ("Assumptions & free parameters": S,
the count of shared k-means patterns, is 64; 15 centroids per pattern).  The
paper names a weighting of the k-means by activations but never defines it
(referee report, minor comment 4); unweighted k-means is used.

Reading: learning has two levels.  (1) Each normalised group's 127 non-scale
values are clustered into 15 clusters with exact one-dimensional k-means (the
textbook dynamic programme over sorted values; optimal clusters are contiguous
runs of the sorted values).  (2) The resulting sorted 15-vectors are clustered
into 64 patterns with Lloyd's algorithm from a k-means++ start.
"""

import numpy as np


def kmeans_1d_exact(values, k):
    """Optimal 1-D k-means of each row of `values` ([G, n], float64).

    Returns (centers [G, k] sorted ascending, sse [G]).  dp[c][i] is the least
    sum of squared errors of the first i sorted values split into c runs; the
    cost of a run is computed from prefix sums.  Vectorised over rows only.
    """
    v = np.sort(np.asarray(values, dtype=np.float64), axis=1)
    G, n = v.shape
    if n < k:
        raise ValueError("need at least k values")
    ps = np.concatenate([np.zeros((G, 1)), np.cumsum(v, axis=1)], axis=1)
    ps2 = np.concatenate([np.zeros((G, 1)), np.cumsum(v * v, axis=1)], axis=1)

    INF = np.inf
    dp = np.full((k + 1, G, n + 1), INF)
    arg = np.zeros((k + 1, G, n + 1), dtype=np.int64)
    dp[0, :, 0] = 0.0
    rows = np.arange(G)
    for c in range(1, k + 1):
        for i in range(c, n - (k - c) + 1):
            # last run holds sorted values j..i-1, j = c-1 .. i-1
            cnt = i - np.arange(c - 1, i, dtype=np.float64)
            s = ps[:, i:i + 1] - ps[:, c - 1:i]
            s2 = ps2[:, i:i + 1] - ps2[:, c - 1:i]
            cost = np.maximum(s2 - s * s / cnt, 0.0)
            tot = dp[c - 1][:, c - 1:i] + cost
            best = np.argmin(tot, axis=1)
            dp[c][:, i] = tot[rows, best]
            arg[c][:, i] = c - 1 + best
    # recover runs
    centers = np.zeros((G, k))
    i = np.full(G, n)
    for c in range(k, 0, -1):
        j = arg[c][np.arange(G), i]
        cnt = (i - j).astype(np.float64)
        s = ps[np.arange(G), i] - ps[np.arange(G), j]
        centers[:, c - 1] = s / cnt
        i = j
    return centers, dp[k][:, n]


def sse_of_assignment(points, centers, assign):
    d = points - centers[assign]
    return float(np.sum(d * d))


def kmeans_pp_init(points, K, rng):
    """k-means++ seeding (Arthur & Vassilvitskii 2007)."""
    N = points.shape[0]
    idx = [int(rng.integers(N))]
    d2 = np.sum((points - points[idx[0]]) ** 2, axis=1)
    for _ in range(1, K):
        tot = d2.sum()
        if tot <= 0:
            nxt = int(rng.integers(N))
        else:
            nxt = int(rng.choice(N, p=d2 / tot))
        idx.append(nxt)
        d2 = np.minimum(d2, np.sum((points - points[nxt]) ** 2, axis=1))
    return points[idx].copy()


def assign_nearest(points, centers):
    d2 = (np.sum(points * points, axis=1)[:, None]
          - 2.0 * points @ centers.T + np.sum(centers * centers, axis=1)[None, :])
    return np.argmin(d2, axis=1)


def lloyd(points, K, iters, seed, return_history=False):
    """Lloyd's k-means with k-means++ start.

    An empty cluster is re-seeded to the point farthest from its center.
    Returns (centers [K, D], assign [N]) and, if asked, the objective after
    every iteration (non-increasing).
    """
    points = np.asarray(points, dtype=np.float64)
    rng = np.random.default_rng(seed)
    centers = kmeans_pp_init(points, K, rng)
    hist = []
    assign = assign_nearest(points, centers)
    for _ in range(iters):
        new = centers.copy()
        for c in range(K):
            m = assign == c
            if np.any(m):
                new[c] = points[m].mean(axis=0)
        d = np.sum((points - new[assign]) ** 2, axis=1)
        for c in range(K):
            if not np.any(assign == c):
                far = int(np.argmax(d))
                new[c] = points[far]
                d[far] = 0.0
        centers = new
        assign = assign_nearest(points, centers)
        hist.append(sse_of_assignment(points, centers, assign))
        if len(hist) >= 2 and hist[-1] == hist[-2]:
            break
    if return_history:
        return centers, assign, hist
    return centers, assign
