"""Pins of the reference k-means and cluster order (no GPU)."""

import os

import numpy as np
import pytest

from oracle import kmeans as ok

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _seed_cases():
    with open(os.path.join(GOLDEN, "kmeanspp_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                pts, us, seeds = (s.strip() for s in line.split("|"))
                yield (np.array([[float(p)] for p in pts.split()]),
                       np.array([float(u) for u in us.split()]),
                       [int(s) for s in seeds.split()])


@pytest.mark.parametrize("x,u,seeds", list(_seed_cases()))
def test_seeding_golden(x, u, seeds):
    assert ok.kmeanspp_seeds(x, len(u), u).tolist() == seeds


def test_seeding_frequencies_follow_d2():
    # Over a fine grid of uniforms, each point is chosen as the second seed in
    # proportion to its squared distance from the first.
    rng = np.random.default_rng(20)
    x = rng.normal(size=(9, 3))
    d2 = ((x - x[4]) ** 2).sum(1)
    m = 20000
    counts = np.zeros(9)
    for j in range(m):
        s = ok.kmeanspp_seeds(x, 2, np.array([4.5 / 9, (j + 0.5) / m]))
        counts[s[1]] += 1
    np.testing.assert_allclose(counts / m, d2 / d2.sum(), atol=2.0 / m)


def test_separated_clusters_recovered():
    rng = np.random.default_rng(21)
    centers = np.array([[0.0, 0.0], [100.0, 0.0], [0.0, 100.0], [100.0, 100.0]])
    lab = rng.integers(0, 4, 400)
    x = centers[lab] + rng.normal(scale=1.0, size=(400, 2))
    cent, a, sizes, seeds, hist = ok.kmeans(x, 4, 5, rng.random(4))
    # same partition up to relabelling
    mapping = {}
    for i in range(400):
        mapping.setdefault(lab[i], a[i])
        assert mapping[lab[i]] == a[i]
    assert len(set(mapping.values())) == 4
    for c in range(4):
        np.testing.assert_allclose(cent[c], x[a == c].mean(0), rtol=1e-12)


def test_single_cluster_is_global_mean_and_invariants():
    rng = np.random.default_rng(22)
    x = rng.normal(size=(300, 8)) * rng.uniform(0.5, 3, size=8)
    cent, a, sizes, seeds, hist = ok.kmeans(x, 1, 3, np.array([0.3]))
    np.testing.assert_allclose(cent[0], x.mean(0), rtol=1e-12)
    cent, a, sizes, seeds, hist = ok.kmeans(x, 12, 10, rng.random(12))
    assert all(h2 <= h1 * (1 + 1e-12) for h1, h2 in zip(hist, hist[1:]))
    assert sizes.sum() == 300 and (np.bincount(a, minlength=12) == sizes).all()
    for c in range(12):
        if sizes[c]:
            np.testing.assert_allclose(cent[c], x[a == c].mean(0), rtol=1e-12)
    # at a fixed point (enough rounds) every point is nearest to its own centroid
    cent, a, sizes, seeds, hist = ok.kmeans(x, 12, 200, rng.random(12))
    assert ok.assign(x, cent).tolist() == a.tolist()
    d = ok.sq_dists(x, cent)
    assert (d[np.arange(300), a] <= d.min(1) * (1 + 1e-12) + 1e-12).all()


def test_cluster_order_is_stable_sort():
    rng = np.random.default_rng(23)
    a = rng.integers(0, 7, 100)
    perm, start, size = ok.cluster_order(a, 9, N=104)
    assert sorted(perm.tolist()) == list(range(104))
    assert (perm[100:] == np.arange(100, 104)).all()
    assert (size == np.bincount(a, minlength=9)).all()
    for c in range(9):
        seg = perm[start[c]:start[c] + size[c]]
        assert (a[seg] == c).all() and (np.diff(seg) > 0).all()


# ----------------------------------------------------------- warm start

def _warm_cases():
    with open(os.path.join(GOLDEN, "kmeans_warm_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                p, c, it, tol, a, cf, ch = (s.split() for s in line.split("|"))
                yield ([float(v) for v in p], [float(v) for v in c], int(it[0]), int(tol[0]),
                       [int(v) for v in a], [float(v) for v in cf], [int(v) for v in ch])


@pytest.mark.parametrize("pts,start,iters,tol,a,cent,changes", list(_warm_cases()))
def test_warm_start_golden(pts, start, iters, tol, a, cent, changes):
    x = np.array(pts)[:, None]
    c, got_a, sizes, got_ch = ok.kmeans_warm(x, np.array(start)[:, None], iters, tol)
    assert got_a.tolist() == a and got_ch.tolist() == changes
    np.testing.assert_allclose(c[:, 0], cent, rtol=0, atol=1e-12)
    assert sizes.tolist() == np.bincount(a, minlength=len(start)).tolist()


def test_cold_run_is_warm_start_from_its_seeds():
    rng = np.random.default_rng(21)
    x = np.concatenate([rng.normal(m, 1.0, size=(60, 3)) for m in (0.0, 4.0, 9.0, 15.0)])
    u = rng.random(6)
    for iters in (1, 3, 12):
        c, a, s, seeds, _ = ok.kmeans(x, 6, iters, u)
        cw, aw, sw, ch = ok.kmeans_warm(x, x[seeds], iters)
        assert np.array_equal(a, aw) and np.array_equal(s, sw)
        np.testing.assert_array_equal(c, cw)
        assert ch[0] == len(x)


def test_converged_centroids_are_a_fixed_point():
    rng = np.random.default_rng(22)
    x = rng.normal(size=(300, 4))
    c, a, s, ch = ok.kmeans_warm(x, x[:8], 200)
    stop = int(np.argmax(ch == 0))
    assert ch[stop] == 0 and (ch[stop:] == 0).all() and (ch[1:stop] > 0).all()
    c2, a2, s2, ch2 = ok.kmeans_warm(x, c, 5)
    assert ch2.tolist() == [300, 0, 0, 0, 0]
    np.testing.assert_array_equal(c2, c)
    assert np.array_equal(a2, a) and np.array_equal(s2, s)


# ------------------------------------------------------- empty clusters

def _empty_cases():
    with open(os.path.join(GOLDEN, "kmeans_empty_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield [s.split() for s in line.split("|")]


@pytest.mark.parametrize("case", list(_empty_cases()))
def test_empty_cluster_keeps_its_centroid_golden(case):
    kind = case[0][0]
    x = np.array([float(v) for v in case[1]])[:, None]
    if kind == "warm":
        start, iters, tol, a, cent, sizes, changes = case[2:]
        c, got_a, got_s, got_ch = ok.kmeans_warm(x, np.array([float(v) for v in start])[:, None],
                                                 int(iters[0]), int(tol[0]))
        assert got_ch.tolist() == [int(v) for v in changes]
        # one round of the update from the start also leaves the empty centroids
        a0 = ok.assign(x, np.array([float(v) for v in start])[:, None])
        c1, s1 = ok.update(x, a0, np.array([float(v) for v in start])[:, None])
        for j, n in enumerate(s1):
            if n == 0:
                assert c1[j, 0] == float(start[j])
    else:
        u, iters, a, cent, sizes, seeds = case[2:]
        c, got_a, got_s, got_seeds, _ = ok.kmeans(x, len(u), int(iters[0]), np.array([float(v) for v in u]))
        assert got_seeds.tolist() == [int(v) for v in seeds]
    assert got_a.tolist() == [int(v) for v in a]
    assert got_s.tolist() == [int(v) for v in sizes]
    np.testing.assert_allclose(c[:, 0], [float(v) for v in cent], rtol=0, atol=1e-12)
