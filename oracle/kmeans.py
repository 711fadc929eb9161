"""k-means clustering and cluster-contiguous order (CPU reference, test infrastructure).

Sparse VideoGen2 summary, Metodologia A ("Clustering", "Permutazione"): the
query and key vectors of a head are clustered independently with k-means and
tokens are permuted so that each cluster is contiguous.

Readings where the pages are silent: squared Euclidean distance on the raw
vectors; k-means++ seeding (Arthur & Vassilvitskii, 2007) driven by uniforms
passed in by the caller; ties go to the lower cluster index; an empty cluster
keeps its previous centroid; ``iters`` rounds of (assign, update); the output
clustering is the last assignment and the centroids are its cluster means.

Pins (tests/test_oracle_kmeans.py): well-separated hand-made clusters are
recovered exactly; C = 1 gives the global mean; inertia never increases over
Lloyd rounds; final centroids are the means of their members; every point is
nearest to its own centroid; seeding follows the D^2 inverse-CDF rule
(checked against a brute-force loop); the cluster order is a stable sort;
``kmeans_warm`` -- a hand-worked 1-D case (tests/golden/kmeans_warm_cases.txt),
a cold run equals a warm start from its seeds, converged centroids are a
fixed point; empty clusters -- hand-worked rounds in which a cluster gets no
point and keeps its centroid (tests/golden/kmeans_empty_cases.txt).
"""

from __future__ import annotations

import numpy as np


def sq_dists(x: np.ndarray, c: np.ndarray) -> np.ndarray:
    """||x_i - c_j||^2 for all pairs, float64 [n, C]."""
    x = np.asarray(x, np.float64)
    c = np.asarray(c, np.float64)
    d = (x * x).sum(1)[:, None] - 2.0 * (x @ c.T) + (c * c).sum(1)[None, :]
    return np.maximum(d, 0.0)


def kmeanspp_seeds(x: np.ndarray, C: int, u: np.ndarray) -> np.ndarray:
    """Indices of the C k-means++ seeds, using the uniforms u[0..C-1].

    First seed: index floor(u0 * n). Each next seed is drawn with probability
    proportional to D^2 (squared distance to the nearest seed so far) by
    inverse CDF over token order: the first index whose inclusive running sum
    of D^2 exceeds u_r * sum(D^2).
    """
    x = np.asarray(x, np.float64)
    n = x.shape[0]
    seeds = [min(int(np.floor(float(u[0]) * n)), n - 1)]
    d2 = ((x - x[seeds[0]]) ** 2).sum(1)
    for r in range(1, C):
        total = d2.sum()
        if total <= 0.0:
            i = min(int(np.floor(float(u[r]) * n)), n - 1)
        else:
            c = np.cumsum(d2)
            i = int(np.searchsorted(c, float(u[r]) * total, side="right"))
            i = min(i, n - 1)
        seeds.append(i)
        d2 = np.minimum(d2, ((x - x[i]) ** 2).sum(1))
    return np.asarray(seeds, dtype=np.int64)


def assign(x: np.ndarray, cent: np.ndarray) -> np.ndarray:
    """Nearest centroid of every point (ties -> lower index)."""
    return np.argmin(sq_dists(x, cent), axis=1).astype(np.int64)


def update(x: np.ndarray, a: np.ndarray, prev: np.ndarray):
    """Cluster means; an empty cluster keeps ``prev``. Returns (cent, sizes)."""
    x = np.asarray(x, np.float64)
    C = prev.shape[0]
    sizes = np.bincount(a, minlength=C).astype(np.int64)
    cent = np.array(prev, dtype=np.float64, copy=True)
    for c in range(C):
        if sizes[c] > 0:
            cent[c] = x[a == c].mean(axis=0)
    return cent, sizes


def inertia(x, a, cent) -> float:
    x = np.asarray(x, np.float64)
    return float(((x - np.asarray(cent, np.float64)[a]) ** 2).sum())


def kmeans(x: np.ndarray, C: int, iters: int, u: np.ndarray):
    """k-means++ seeding then ``iters`` Lloyd rounds.

    Returns (centroids float64 [C, d], assignment int64 [n], sizes int64 [C],
    seeds int64 [C], inertia after each round list[float]).
    """
    x = np.asarray(x, np.float64)
    seeds = kmeanspp_seeds(x, C, u)
    cent = x[seeds].copy()
    a = np.zeros(x.shape[0], dtype=np.int64)
    sizes = np.zeros(C, dtype=np.int64)
    hist = []
    for _ in range(iters):
        a = assign(x, cent)
        cent, sizes = update(x, a, cent)
        hist.append(inertia(x, a, cent))
    return cent, a, sizes, seeds, hist


def kmeans_warm(x: np.ndarray, cent0: np.ndarray, max_iters: int, tol_moves: int = 0):
    """Lloyd rounds started from given centroids, stopping once (nearly) settled.

    Sparse VideoGen2 summary, Metodologia C.1 ("Cache dei Centroidi"): the
    centroids of the previous denoising step initialise k-means at the next
    step, so no seeding is done. Each round assigns every point to its nearest
    centroid and moves the centroids to the cluster means (``assign`` and
    ``update`` above). ``changes[t]`` is the number of points whose assignment
    differs from round t - 1 (round 0 counts all points). The loop stops after
    the first round that moves at most ``tol_moves`` points (its update is
    kept) and the remaining entries are 0. With tol_moves = 0 that round moved
    nothing, so it left the centroids where they were and every later round
    would repeat it: the result is the fixed point.

    Returns (centroids float64 [C, d], assignment int64 [n], sizes int64 [C],
    changes int64 [max_iters]).
    """
    x = np.asarray(x, np.float64)
    cent = np.array(cent0, dtype=np.float64, copy=True)
    n = x.shape[0]
    changes = np.zeros(max_iters, dtype=np.int64)
    a_prev = None
    a = np.zeros(n, dtype=np.int64)
    sizes = np.zeros(cent.shape[0], dtype=np.int64)
    for t in range(max_iters):
        a = assign(x, cent)
        changes[t] = n if a_prev is None else int((a != a_prev).sum())
        cent, sizes = update(x, a, cent)
        if changes[t] <= tol_moves:
            break
        a_prev = a
    return cent, a, sizes, changes


def cluster_order(a: np.ndarray, C: int, N: int | None = None):
    """Stable order grouping tokens by cluster.

    Returns perm int64 [N] (perm[new] = old index; positions past the
    clustered tokens map to themselves), start int64 [C], size int64 [C].
    """
    a = np.asarray(a, dtype=np.int64)
    n = a.shape[0]
    N = n if N is None else N
    perm = np.argsort(a, kind="stable")
    size = np.bincount(a, minlength=C).astype(np.int64)
    start = np.concatenate([[0], np.cumsum(size)[:-1]]).astype(np.int64)
    perm = np.concatenate([perm, np.arange(n, N)]).astype(np.int64)
    return perm, start, size
