"""Pins of the mask-quality diagnostic reference (no GPU)."""

import os

import numpy as np
import pytest
import torch

from oracle import diagnostic as od
from oracle import layout as ol
from oracle import mask as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_row_masses_sum_to_row_counts_and_ordering():
    rng = np.random.default_rng(30)
    q, k = 2 * rng.normal(size=(150, 16)), 2 * rng.normal(size=(150, 16))
    st, ln = ol.raster_blocks(150, 32)
    tmax, tsum, tmin = od.tile_stats(q, k, st, ln, st, ln)
    np.testing.assert_allclose(tsum.sum(1), ln, rtol=1e-12)
    area = ln[:, None] * ln[None, :]
    assert (tmax >= tsum / area - 1e-15).all() and (tsum / area >= tmin - 1e-15).all()
    assert (tmin > 0).all()


def test_one_token_tiles_are_the_softmax_matrix():
    rng = np.random.default_rng(31)
    q, k = rng.normal(size=(9, 8)), rng.normal(size=(11, 8))
    one_q, one_k = (np.arange(9), np.ones(9, int)), (np.arange(11), np.ones(11, int))
    tmax, tsum, tmin = od.tile_stats(q, k, *one_q, *one_k, scale=0.7)
    ref = torch.softmax(0.7 * torch.from_numpy(q) @ torch.from_numpy(k).T, dim=1).numpy()
    for t in (tmax, tsum, tmin):
        np.testing.assert_allclose(t, ref, rtol=1e-12)


def test_identical_keys_give_uniform_statistics():
    rng = np.random.default_rng(32)
    q = rng.normal(size=(40, 8))
    k = np.tile(rng.normal(size=(1, 8)), (40, 1))
    st, ln = ol.raster_blocks(40, 16)
    tmax, tsum, tmin = od.tile_stats(q, k, st, ln, st, ln)
    np.testing.assert_allclose(tmax, 1 / 40, rtol=1e-12)
    np.testing.assert_allclose(tmin, 1 / 40, rtol=1e-12)
    np.testing.assert_allclose(tsum, ln[:, None] * ln[None, :] / 40, rtol=1e-12)


def _cases():
    with open(os.path.join(GOLDEN, "mask_recall_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                a, b, c, r, m = (x.split() for x in line.split("|"))
                yield ([float(v) for v in a], [float(v) for v in b], [int(v) for v in c], float(r[0]),
                       float(m[0]))


@pytest.mark.parametrize("tmax,tsum,kept,rec,mass", list(_cases()))
def test_recall_golden(tmax, tsum, kept, rec, mass):
    keep = np.zeros((1, len(tmax)), dtype=bool)
    keep[0, kept] = True
    r, m = od.mask_recall(keep, np.array([tmax]), np.array([tsum]))
    assert r[0] == pytest.approx(rec, abs=1e-15) and m[0] == pytest.approx(mass, abs=1e-15)


def test_oracle_and_full_masks_score_one():
    rng = np.random.default_rng(33)
    q, k = 3 * rng.normal(size=(128, 16)), 3 * rng.normal(size=(128, 16))
    st, ln = ol.raster_blocks(128, 16)
    tmax, tsum, _ = od.tile_stats(q, k, st, ln, st, ln)
    keep, _ = om.block_mask(q, k, st, ln, st, ln, 0.3)
    orc = od.oracle_mask(tmax, keep.sum(1))
    r, m = od.mask_recall(orc, tmax, tsum)
    assert (r == 1).all()
    r, m = od.mask_recall(np.ones_like(keep), tmax, tsum)
    assert (r == 1).all() and np.allclose(m, 1, rtol=1e-12)
    r, m = od.mask_recall(keep, tmax, tsum)
    assert ((0 <= r) & (r <= 1)).all() and ((0 < m) & (m <= 1 + 1e-12)).all()
