"""Mask comparison with a tolerance band around the CDF threshold.

A GPU bit may differ from the reference only where the reference's own
numbers leave the decision open: the block's cumulative mass lies within
``delta`` of thr, counting blocks whose probabilities are within relative
``rho`` of it as possibly lighter or heavier (ties under rounding).

On a mask without a window the kept set as a whole is checked too (NABLA
summary, Metodologia section 2, "CDF Thresholding": the kept blocks are the
heaviest ones that carry the row's cumulative mass past 1 - thr). With p the
row's normalised reference probabilities and K the GPU's kept set:
  * enough mass:   mass(K) > 1 - thr - delta;
  * nothing spare: mass(K) - min_{J in K} p_J <= 1 - thr + delta;
  * heaviest:      every dropped p <= every kept p * (1 + rho).
These catch a mask that moves every in-band bit the same way, which the
per-bit rule alone would accept.
"""

import numpy as np


def sure_bits(p: np.ndarray, thr: float, rho: float = 1e-4, delta: float = 1e-4):
    """(sure_keep, sure_drop) bool arrays for one row of probabilities."""
    p = np.asarray(p, np.float64)
    p = p / p.sum()
    s = np.sort(p)
    c = np.concatenate([[0.0], np.cumsum(s)])
    lo = np.searchsorted(s, p * (1 - rho), side="left")     # count of p_K < p_J(1-rho)
    hi = np.searchsorted(s, p * (1 + rho), side="right")    # count of p_K <= p_J(1+rho)
    L = c[lo]
    U = c[hi]
    sure_drop = U < thr - delta
    sure_keep = (L + p) >= thr + delta
    return sure_keep, sure_drop


def set_violations(p: np.ndarray, thr: float, keep: np.ndarray, rho: float = 1e-4,
                   delta: float = 1e-4) -> int:
    """Number of the three set-level properties (see the module text) that one
    window-free row's kept set breaks (0..3)."""
    p = np.asarray(p, np.float64)
    p = p / p.sum()
    keep = np.asarray(keep, dtype=bool)
    if not keep.any():
        return 1                        # the heaviest block is always kept
    mass = float(p[keep].sum())
    bad = 0
    if not mass > 1.0 - thr - delta:
        bad += 1
    if not mass - float(p[keep].min()) <= 1.0 - thr + delta:
        bad += 1
    if (~keep).any() and not float(p[~keep].max()) <= float(p[keep].min()) * (1.0 + rho):
        bad += 1
    return bad


def mask_mismatches(P: np.ndarray, thr: float, gpu_keep: np.ndarray, window=None,
                    rho: float = 1e-4, delta: float = 1e-4, valid_cols=None):
    """Sure bits where gpu_keep disagrees, over all rows of P, plus (without a
    window) the set-level properties each row's kept set breaks."""
    bad = 0
    for i in range(P.shape[0]):
        cols = slice(None) if valid_cols is None else valid_cols
        k, d = sure_bits(P[i][cols], thr, rho, delta)
        g = gpu_keep[i][cols]
        if window is not None:
            w = window[i][cols]
            k = k | w
            d = d & ~w
        else:
            bad += set_violations(P[i][cols], thr, g, rho, delta)
        bad += int(((k & ~g) | (d & g)).sum())
    return bad


def keep_from_lists(kv_count: np.ndarray, kv_index: np.ndarray, nkb: int) -> np.ndarray:
    """bool [rows, nkb] from (count, ascending index) lists; checks the lists."""
    rows = kv_count.shape[0]
    keep = np.zeros((rows, nkb), dtype=bool)
    for r in range(rows):
        ids = kv_index[r, :kv_count[r]]
        assert (ids >= 0).all() and (ids < nkb).all(), r
        assert (np.diff(ids) > 0).all(), r
        keep[r, ids] = True
    return keep
