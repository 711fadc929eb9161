"""Mask-quality diagnostic (CPU reference, test infrastructure).

Veda summary, section 2.1 ("Punteggio dei Tile Distillato"): the reference
("oracle") tile mask is built by max-pooling the full attention matrix over
each query-tile x key-tile region, and tile descriptors carry the mean,
maximum and minimum of a tile (TripPool). Section 3 ties generation quality to
how well a sparse mask aligns with that tile geometry of the full attention.
The ground truth takes two passes: the row normalisers of the full
attention, then the pooled map.

Readings (no trained estimator here): the statistics are taken of the full
attention probabilities P (softmax over every valid key of a query row, scale
1/sqrt(d)) over the valid (query, key) pairs of each tile: max, sum (the
tile's attention mass; mean = sum / area) and min. A mask is scored two ways
per query block I that keeps k_I tiles:
  * oracle recall: the share of the k_I tiles with the largest max-pooled
    value (ties: the lower key-block index ranks higher) that the mask keeps;
  * mass recall: the share of the row block's attention mass inside its kept
    tiles.

Pins (tests/test_oracle_diagnostic.py): every row's mass sums to its row
count; one-token tiles give the softmax matrix itself (torch, float64);
identical keys give uniform statistics; max >= mean >= min; a mask equal to
its own oracle mask, or keeping everything, scores 1; a hand-worked case
(tests/golden/mask_recall_cases.txt).
"""

from __future__ import annotations

import numpy as np


def full_attention_probs(q: np.ndarray, k: np.ndarray, scale: float | None = None) -> np.ndarray:
    """P = softmax(scale * q k^T) over all keys, float64 [n_q, n_k]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    scale = 1.0 / np.sqrt(q.shape[1]) if scale is None else scale
    s = scale * (q @ k.T)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def tile_stats(q, k, qstart, qlen, kstart, klen, scale: float | None = None):
    """Max, sum and min of the full attention over every (query block, key block)
    tile. q, k: [n, d] valid tokens; blocks are (start, length) arrays.
    Returns three float64 [nq, nk] arrays; a tile with no pairs gives 0, 0, 0.
    """
    P = full_attention_probs(q, k, scale)
    nq, nk = len(qstart), len(kstart)
    tmax = np.zeros((nq, nk))
    tsum = np.zeros((nq, nk))
    tmin = np.zeros((nq, nk))
    for I in range(nq):
        rows = slice(int(qstart[I]), int(qstart[I]) + int(qlen[I]))
        for J in range(nk):
            t = P[rows, int(kstart[J]):int(kstart[J]) + int(klen[J])]
            if t.size:
                tmax[I, J], tsum[I, J], tmin[I, J] = t.max(), t.sum(), t.min()
    return tmax, tsum, tmin


def oracle_mask(tmax: np.ndarray, counts: np.ndarray) -> np.ndarray:
    """Per row I, the counts[I] tiles with the largest max-pooled value (ties:
    lower index first). bool [nq, nk]."""
    nq, nk = tmax.shape
    out = np.zeros((nq, nk), dtype=bool)
    for I in range(nq):
        order = np.lexsort((np.arange(nk), -tmax[I]))      # value descending, then index ascending
        out[I, order[:int(counts[I])]] = True
    return out


def mask_recall(keep: np.ndarray, tmax: np.ndarray, tsum: np.ndarray):
    """Per query block: (oracle recall, mass recall) float64 [nq] each.

    Rows that keep nothing score 0 oracle recall; rows with no attention mass
    (padding) score 0 mass recall.
    """
    keep = np.asarray(keep, dtype=bool)
    k = keep.sum(1)
    orc = oracle_mask(tmax, k)
    hit = (keep & orc).sum(1)
    rec = np.where(k > 0, hit / np.maximum(k, 1), 0.0)
    tot = tsum.sum(1)
    mass = np.where(tot > 0, (tsum * keep).sum(1) / np.where(tot > 0, tot, 1.0), 0.0)
    return rec, mass
