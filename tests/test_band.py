"""The mask comparison rule itself (tests/band.py), on the CPU.

NABLA summary, Metodologia section 2, "CDF Thresholding": the kept blocks are
the heaviest ones that carry the row's cumulative mass past 1 - thr. The
comparison must accept the reference's own masks and reject masks that are
wrong in ways the per-bit band alone would let through.
"""

import numpy as np

from oracle import mask as om
from tests.band import mask_mismatches, set_violations, sure_bits


def _rows(seed, n_rows=40, n=300):
    rng = np.random.default_rng(seed)
    s = rng.normal(size=(n_rows, n)) * rng.uniform(0.5, 4.0, size=(n_rows, 1))
    return om.softmax_rows(s)


def test_reference_masks_pass():
    for thr in (0.0, 0.1, 0.5, 0.9, 1.0):
        P = _rows(1)
        keep = om.cdf_mask(P, thr)
        assert mask_mismatches(P, thr, keep) == 0
        assert all(set_violations(p, thr, k) == 0 for p, k in zip(P, keep))


def test_wide_band_flipped_one_way_is_caught():
    # One heavy block and twenty tied ones: with thr = 0.2 the cut falls inside
    # the ties, so every tied block is in the band and the per-bit rule accepts
    # any choice among them. Keeping all of them, or none, breaks the set rule.
    p = np.array([0.5] + [0.025] * 20)
    thr = 0.2
    ref = om.cdf_keep(p, thr)
    assert mask_mismatches(p[None], thr, ref[None]) == 0
    k, d = sure_bits(p, thr)
    assert k[0] and not k[1:].any() and not d.any()     # the ties are all in the band
    all_kept = np.ones(21, dtype=bool)
    none_kept = np.zeros(21, dtype=bool)
    none_kept[0] = True
    for g in (all_kept, none_kept):
        # the per-bit rule alone accepts it ...
        kk, dd = sure_bits(p, thr)
        assert not ((kk & ~g) | (dd & g)).any()
        # ... the set-level rule does not
        assert set_violations(p, thr, g) > 0
        assert mask_mismatches(p[None], thr, g[None]) > 0


def test_every_band_bit_flipped_is_caught_on_real_rows():
    # Rows with many near-ties at the cut: a mask that sets (or clears) every
    # in-band bit fails, the reference's own mask passes.
    rng = np.random.default_rng(5)
    caught = 0
    for _ in range(50):
        base = rng.uniform(0.5, 1.0, size=6)
        ties = np.full(60, rng.uniform(0.01, 0.02))
        ties *= 1 + rng.uniform(-5e-6, 5e-6, size=60)      # within rho of each other
        p = np.concatenate([base, ties])
        p /= p.sum()
        thr = float(rng.uniform(0.05, 0.2))
        ref = om.cdf_keep(p, thr)
        assert set_violations(p, thr, ref) == 0
        k, d = sure_bits(p, thr)
        band = ~k & ~d
        if band.sum() < 4:
            continue
        for val in (True, False):
            g = ref.copy()
            g[band] = val
            assert mask_mismatches(p[None], thr, g[None]) > 0
        caught += 1
    assert caught >= 20


def test_heaviest_rule_catches_swapped_blocks():
    # keep a light block in place of a heavy one with the same total count
    p = np.array([0.4, 0.3, 0.2, 0.06, 0.04])
    ref = om.cdf_keep(p, 0.15)
    assert ref.tolist() == [True, True, True, False, False]
    g = np.array([True, True, False, True, True])
    assert set_violations(p, 0.15, g) > 0
    assert set_violations(p, 0.15, np.zeros(5, dtype=bool)) > 0
