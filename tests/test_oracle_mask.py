"""Pins of the CPU reference mask stage against closed forms, brute force and
hand-worked fixtures (no GPU)."""

import itertools
import os

import numpy as np
import pytest

from oracle import mask as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cases(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def _cdf_cases():
    out = []
    for line in _cases("cdf_select_cases.txt"):
        thr, vals, kept = (s.strip() for s in line.split("|"))
        out.append((float(thr), np.array([float(v) for v in vals.split()]),
                    sorted(int(i) for i in kept.split())))
    return out


# ---------------------------------------------------------------- pooling

def test_pool_golden():
    xs, blocks, means = [], [], []
    for line in _cases("pool_cases.txt"):
        tag, vals = line.split(":")
        vals = [float(v) for v in vals.split()]
        {"x": xs, "block": blocks, "mean": means}[tag].append(vals)
    x = np.array(xs)
    st = np.array([int(b[0]) for b in blocks])
    ln = np.array([int(b[1]) for b in blocks])
    np.testing.assert_array_equal(om.pool(x, st, ln), np.array(means))


def test_pool_constant_blocks_and_linearity():
    rng = np.random.default_rng(1)
    st = np.array([0, 64, 128, 150])
    ln = np.array([64, 64, 22, 7])
    vals = rng.normal(size=(4, 16))
    x = np.concatenate([np.repeat(vals[i:i + 1], ln[i], axis=0) for i in range(4)])
    np.testing.assert_allclose(om.pool(x, st, ln), vals, rtol=1e-14, atol=0)
    a = rng.normal(size=(157, 16))
    b = rng.normal(size=(157, 16))
    np.testing.assert_allclose(om.pool(2.0 * a - 3.0 * b, st, ln),
                               2.0 * om.pool(a, st, ln) - 3.0 * om.pool(b, st, ln),
                               atol=1e-13)


# ---------------------------------------------------------- reduced attention

def test_reduced_two_blocks_is_logistic():
    # Two key blocks: the probability of block 0 is the logistic of the score gap.
    rng = np.random.default_rng(2)
    qbar = rng.normal(size=(5, 8))
    kbar = rng.normal(size=(2, 8))
    scale = 0.37
    p = om.softmax_rows(om.reduced_scores(qbar, kbar, scale))
    gap = scale * (qbar @ (kbar[0] - kbar[1]))
    np.testing.assert_allclose(p[:, 0], 1.0 / (1.0 + np.exp(-gap)), rtol=1e-13)
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=1e-14)


def test_reduced_identical_keys_uniform():
    rng = np.random.default_rng(3)
    kbar = np.repeat(rng.normal(size=(1, 8)), 7, axis=0)
    p = om.softmax_rows(om.reduced_scores(rng.normal(size=(3, 8)), kbar, 1.0))
    np.testing.assert_allclose(p, 1.0 / 7.0, rtol=1e-14)


def test_log_weight_equals_cluster_splitting():
    # Weighting a key by its size n must equal n identical keys of size one.
    rng = np.random.default_rng(4)
    s = rng.normal(size=(3, 4))
    n = np.array([1, 3, 2, 5])
    w = om.softmax_rows(s, np.log(n))
    expanded = np.repeat(s, n, axis=1)
    pe = om.softmax_rows(expanded)
    grouped = np.add.reduceat(pe, np.concatenate([[0], np.cumsum(n)[:-1]]), axis=1)
    np.testing.assert_allclose(w, grouped, rtol=1e-13)


# ------------------------------------------------------------- CDF select

@pytest.mark.parametrize("thr,row,kept", _cdf_cases())
def test_cdf_golden(thr, row, kept):
    assert sorted(np.nonzero(om.cdf_keep(row, thr))[0].tolist()) == kept


def _brute_force_keep(p, thr):
    """Smallest set whose mass exceeds (1-thr)*Z; among those the heaviest.

    With no such set (thr = 0), every block is kept.
    """
    n = len(p)
    z = p.sum()
    for size in range(1, n + 1):
        best, best_mass = None, -1.0
        for sub in itertools.combinations(range(n), size):
            m = p[list(sub)].sum()
            if m > (1.0 - thr) * z and m > best_mass:
                best, best_mass = sub, m
        if best is not None:
            return set(best)
    return set(range(n))


def test_cdf_brute_force_minimal_heaviest():
    rng = np.random.default_rng(5)
    for trial in range(60):
        n = int(rng.integers(1, 11))
        # heavy-tailed rows like softmax over scores
        p = np.exp(rng.normal(scale=2.0, size=n))
        thr = float(rng.choice([0.05, 0.1, 0.2, 0.35, 0.5, 0.8]))
        got = set(np.nonzero(om.cdf_keep(p, thr))[0].tolist())
        assert got == _brute_force_keep(p, thr), (trial, p, thr)


def test_cdf_invariants_and_special_cases():
    rng = np.random.default_rng(6)
    for _ in range(200):
        n = int(rng.integers(1, 300))
        p = np.exp(rng.normal(scale=3.0, size=n))
        thr = float(rng.uniform(0, 1))
        keep = om.cdf_keep(p, thr)
        z = p.sum()
        km = p[keep].sum()
        assert keep[np.argmax(p)]
        assert km >= (1 - thr) * z * (1 - 1e-12)
        assert km - p[keep].min() <= (1 - thr) * z * (1 + 1e-12)
        if (~keep).any():
            assert p[~keep].max() <= p[keep].min()
        assert om.cdf_keep(p, 0.0).all()
        k1 = om.cdf_keep(p, 1.0)
        assert k1.sum() == 1 and k1[np.argmax(p)]


# Planted mistakes: each variant below differs from the reading in one plausible
# way; the pins above must reject every one of them.

def _variant_desc_tiebreak(p, thr):
    n = len(p)
    order = np.lexsort((np.arange(n), p))      # ties: lower index lighter (wrong)
    c = np.cumsum(p[order])
    keep = np.zeros(n, bool)
    keep[order] = ~(c < thr * c[-1])
    return keep


def _variant_le(p, thr):
    n = len(p)
    order = np.lexsort((-np.arange(n), p))
    c = np.cumsum(p[order])
    keep = np.zeros(n, bool)
    keep[order] = ~(c <= thr * c[-1])          # strictness flipped (wrong)
    return keep


def _variant_keep_tail(p, thr):
    n = len(p)
    order = np.lexsort((-np.arange(n), -p))    # heaviest first, keep where CDF > 1-thr
    c = np.cumsum(p[order])
    keep = np.zeros(n, bool)
    keep[order] = c > (1 - thr) * c[-1]        # literal "exceeds" on a descending CDF
    return keep


@pytest.mark.parametrize("variant", [_variant_desc_tiebreak, _variant_le, _variant_keep_tail])
def test_planted_mistakes_are_caught(variant, monkeypatch):
    caught = False
    for thr, row, kept in _cdf_cases():
        if sorted(np.nonzero(variant(row, thr))[0].tolist()) != kept:
            caught = True
    assert caught, "golden cases did not detect a planted selection mistake"


# ----------------------------------------------------------- block mask

def test_block_mask_thr0_keeps_all_and_window_union():
    rng = np.random.default_rng(7)
    q = rng.normal(size=(200, 16))
    k = rng.normal(size=(200, 16))
    st = np.array([0, 64, 128, 192])
    ln = np.array([64, 64, 64, 8])
    keep, p = om.block_mask(q, k, st, ln, st, ln, 0.0)
    assert keep.all()
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=1e-14)
    win = np.eye(4, dtype=bool)
    keep2, _ = om.block_mask(3 * q, 3 * k, st, ln, st, ln, 0.9, window=win)
    keep3, _ = om.block_mask(3 * q, 3 * k, st, ln, st, ln, 0.9)
    assert (keep2 >= win).all() and (keep2 == (keep3 | win)).all()


def test_centroid_mask_special_cases():
    rng = np.random.default_rng(8)
    cq = rng.normal(size=(6, 16))
    ck = rng.normal(size=(9, 16))
    nq = np.array([3, 0, 5, 2, 2, 1])
    nk = np.array([4, 4, 0, 4, 4, 4, 0, 4, 4])
    keep, w = om.centroid_mask(cq, nq, ck, nk, 1.0)
    assert (keep == ((nq > 0)[:, None] & (nk > 0)[None, :])).all()
    assert (w[:, nk == 0] == 0).all()
    # equal sizes: the weights are the plain softmax over non-empty clusters
    sel = nk > 0
    p = om.softmax_rows(om.reduced_scores(cq, ck[sel], 0.25))
    np.testing.assert_allclose(w[:, sel], p, rtol=1e-13)


def test_block_mask_empty_blocks_take_no_part():
    # inserting blocks with no tokens changes nothing else: they are never kept
    # as key blocks and keep nothing as query blocks (window included)
    rng = np.random.default_rng(17)
    q = 3 * rng.normal(size=(200, 16))
    k = 3 * rng.normal(size=(200, 16))
    st = np.array([0, 64, 128, 192])
    ln = np.array([64, 64, 64, 8])
    pos = [1, 3, 6]                                   # where the empty blocks go
    st2, ln2 = list(st), list(ln)
    for i in pos:
        st2.insert(i, 200)
        ln2.insert(i, 0)
    st2, ln2 = np.array(st2), np.array(ln2)
    real = ln2 > 0
    for thr in (0.0, 0.3, 0.9):
        keep, p = om.block_mask(q, k, st, ln, st, ln, thr)
        keep2, p2 = om.block_mask(q, k, st2, ln2, st2, ln2, thr)
        assert np.array_equal(keep2[np.ix_(real, real)], keep)
        np.testing.assert_allclose(p2[np.ix_(real, real)], p, rtol=1e-13)
        assert not keep2[~real].any() and not keep2[:, ~real].any()
        assert (p2[:, ~real] == 0).all()
    win = np.ones((7, 7), dtype=bool)
    keep3, _ = om.block_mask(q, k, st2, ln2, st2, ln2, 0.9, window=win)
    assert not keep3[~real].any() and keep3[real].all()


# ------------------------------------------------ centroid top-p (size-weighted)

def _num(tok):
    """A fixture number: a decimal, a fraction 'a/b', or 'lnX' / '-lnX'."""
    from fractions import Fraction
    neg = tok.startswith("-")
    t = tok[1:] if neg else tok
    v = float(np.log(float(t[2:]))) if t.startswith("ln") else float(Fraction(t))
    return -v if neg else v


def _rows(field):
    return np.array([[_num(t) for t in r.split()] for r in field.split(";")])


def _centroid_cases():
    with open(os.path.join(GOLDEN, "centroid_mask_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield [s.strip() for s in line.split("|")]


@pytest.mark.parametrize("case", list(_centroid_cases()))
def test_centroid_mask_golden(case):
    scale, cq, nq, ck, nk, p, w, kept = case
    nq = np.array([int(v) for v in nq.split()])
    nk = np.array([int(v) for v in nk.split()])
    keep, got_w = om.centroid_mask(_rows(cq), nq, _rows(ck), nk, float(p), scale=float(scale))
    np.testing.assert_allclose(got_w, _rows(w), rtol=1e-12, atol=1e-15)
    want = np.zeros_like(keep)
    for r, ids in enumerate(kept.split(";")):
        if ids.strip() != "-":
            want[r, [int(i) for i in ids.split()]] = True
    assert np.array_equal(keep, want)


def test_centroid_weight_equals_copies_of_the_centroid():
    # A key cluster of n tokens weighs exactly what n clusters of one token at
    # the same centroid weigh together: the size enters as a factor n_b on
    # exp(s_ab). Checked through centroid_mask on unequal sizes.
    rng = np.random.default_rng(31)
    cq = rng.normal(size=(5, 8))
    ck = rng.normal(size=(7, 8))
    nq = np.array([2, 1, 4, 3, 1])
    nk = np.array([1, 5, 2, 9, 3, 1, 6])
    _, w = om.centroid_mask(cq, nq, ck, nk, 0.9, scale=0.7)
    ck_copies = np.repeat(ck, nk, axis=0)
    owner = np.repeat(np.arange(7), nk)
    _, w1 = om.centroid_mask(cq, nq, ck_copies, np.ones(len(ck_copies), np.int64), 0.9, scale=0.7)
    summed = np.stack([w1[:, owner == b].sum(1) for b in range(7)], axis=1)
    np.testing.assert_allclose(w, summed, rtol=1e-13)
    # and an unweighted softmax differs when sizes differ
    plain = om.softmax_rows(om.reduced_scores(cq, ck, 0.7))
    assert np.abs(plain - w).max() > 1e-2
