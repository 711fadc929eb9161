"""Dynamic block-mask construction (CPU reference, test infrastructure).

Steps follow the NABLA summary, Metodologia section 2 ("Costruzione della
Maschera Adattiva"), in order: average pooling of Q and K into blocks,
reduced attention over the pooled blocks, per-row CDF thresholding, and
(section 3) the union with a static window. ``centroid_mask`` is the
centroid top-p rule of the Sparse VideoGen2 summary (Metodologia B).

Readings where the pages are silent (each listed in the design notes):
  * the reduced map uses the attention scale 1/sqrt(d);
  * the CDF is taken relative to the row's own total, lightest block first;
    among equal probabilities the higher block index counts as lighter;
    a block is dropped exactly when the inclusive cumulative mass up to it
    stays below thr * total. Equivalently the kept set is the smallest
    heaviest-first set whose mass exceeds (1 - thr) * total, so thr = 0 keeps
    every block and the heaviest block is always kept;
  * pooling averages only the real tokens of a block;
  * a block with no tokens (length 0: padding of per-head layouts with
    different block counts) has no average, so it takes no part in the
    reduced attention: it is never kept by the CDF rule as a key block, and
    as a query block it keeps nothing (the window included).

Pins (tests/test_oracle_mask.py): pooling -- constant blocks, linearity, a
hand-worked fixture; reduced map -- two-block logistic closed form, identical
keys give a uniform row; selection -- brute force over every subset for small
rows, hand-worked fixtures in tests/golden/cdf_select_cases.txt, thr = 0 and
thr = 1 special cases; window union -- superset property and closed-form
counts; centroid top-p -- hand-worked size-weighted cases with unequal
cluster sizes, empty clusters and p < 1 (tests/golden/centroid_mask_cases.txt),
and a key cluster of n tokens weighing exactly what n one-token clusters at
its centroid weigh together.
"""

from __future__ import annotations

import numpy as np


def pool(x: np.ndarray, start: np.ndarray, length: np.ndarray) -> np.ndarray:
    """Block means. x: [n, d]; returns float64 [nblocks, d].

    NABLA summary, Metodologia section 2, "Sottocampionamento": Q and K are
    average-pooled over blocks of tokens.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros((len(start), x.shape[1]), dtype=np.float64)
    for i, (s, n) in enumerate(zip(start, length)):
        if n > 0:                       # a block with no tokens stays 0 (never used)
            out[i] = x[s:s + n].sum(axis=0) / n
    return out


def reduced_scores(qbar: np.ndarray, kbar: np.ndarray, scale: float) -> np.ndarray:
    """Scores between pooled blocks, scale * qbar @ kbar^T (float64).

    NABLA summary, Metodologia section 2, "Attenzione Ridotta": a full
    attention map is computed over the pooled block representations.
    """
    return scale * (np.asarray(qbar, np.float64) @ np.asarray(kbar, np.float64).T)


def softmax_rows(s: np.ndarray, logw: np.ndarray | None = None) -> np.ndarray:
    """Row softmax of s (+ optional per-column log-weight), float64.

    Columns whose log-weight is -inf get probability zero.
    """
    s = np.asarray(s, dtype=np.float64)
    if logw is not None:
        s = s + np.asarray(logw, dtype=np.float64)[None, :]
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def cdf_keep(p: np.ndarray, thr: float) -> np.ndarray:
    """Binarise one row of the reduced map by its CDF. Returns bool [n].

    NABLA summary, Metodologia section 2, "CDF Thresholding": a cumulative
    distribution is computed per row and only the blocks that carry the row
    past 1 - thr are kept. Worked out: order the blocks lightest first (ties:
    higher index lighter), take the inclusive running sum c, and drop a block
    exactly when c < thr * (row total).
    """
    p = np.asarray(p, dtype=np.float64)
    n = p.shape[0]
    idx = np.arange(n)
    order = np.lexsort((-idx, p))          # by p ascending, then index descending
    c = np.cumsum(p[order])
    z = c[-1]
    keep_sorted = ~(c < thr * z)
    keep = np.zeros(n, dtype=bool)
    keep[order] = keep_sorted
    return keep


def cdf_mask(p: np.ndarray, thr: float) -> np.ndarray:
    """``cdf_keep`` applied to every row of a [nq, nk] map."""
    return np.stack([cdf_keep(row, thr) for row in np.asarray(p)], axis=0)


def block_mask(q: np.ndarray, k: np.ndarray, qstart, qlen, kstart, klen,
               thr: float, scale: float | None = None,
               window: np.ndarray | None = None):
    """Full mask stage for one head.

    q, k: [n, d] (any float dtype; bf16 values are exact in float64).
    Blocks are (start, length) arrays over the token axis. ``window`` is an
    optional bool [nq, nk] static window OR'd into the CDF mask (NABLA
    summary, Metodologia section 3: M = M_nabla OR M_STA).
    Returns (keep bool [nq, nk], probabilities float64 [nq, nk]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d = q.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    qbar = pool(q, qstart, qlen)
    kbar = pool(k, kstart, klen)
    logw = np.where(np.asarray(klen) > 0, 0.0, -np.inf)
    p = softmax_rows(reduced_scores(qbar, kbar, scale), logw)
    keep = cdf_mask(p, thr)
    keep[:, np.asarray(klen) == 0] = False
    if window is not None:
        keep = keep | window
    keep[np.asarray(qlen) == 0, :] = False
    return keep, p


def centroid_mask(cq: np.ndarray, nq: np.ndarray, ck: np.ndarray, nk: np.ndarray,
                  top_p: float, scale: float | None = None):
    """Centroid top-p selection between query and key clusters.

    Sparse VideoGen2 summary, Metodologia B ("Selezione Top-p Basata sui
    Centroidi"): attention is estimated between cluster centroids, clusters
    are taken heaviest first until the cumulative score reaches p.
    Reading: the estimate of key cluster b for query cluster a is the
    size-weighted softmax w_ab = n_b exp(s_ab) / sum_b' n_b' exp(s_ab'),
    s = scale * c_a . c_b; selection is ``cdf_keep`` with thr = 1 - p; empty
    key clusters are never kept and empty query clusters keep nothing.
    Returns (keep bool [Cq, Ck], w float64 [Cq, Ck]).
    """
    cq = np.asarray(cq, np.float64)
    ck = np.asarray(ck, np.float64)
    nq = np.asarray(nq)
    nk = np.asarray(nk)
    d = cq.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    with np.errstate(divide="ignore"):
        logw = np.where(nk > 0, np.log(np.maximum(nk, 1).astype(np.float64)), -np.inf)
    w = softmax_rows(reduced_scores(cq, ck, scale), logw)
    keep = cdf_mask(w, 1.0 - top_p) & (nk > 0)[None, :] & (nq > 0)[:, None]
    return keep, w
