"""Pins of the reference layouts and window (no GPU)."""

import os

import numpy as np
import pytest

from gen import token_coords
from oracle import layout as ol

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_raster_blocks_closed_form():
    st, ln = ol.raster_blocks(32760, 64)
    assert len(st) == 512 and ln[-1] == 32760 - 511 * 64 == 56
    assert (ln[:-1] == 64).all() and (st == 64 * np.arange(512)).all()
    st, ln = ol.raster_blocks(118800, 64)
    assert len(st) == 1857 and ln[-1] == 16


@pytest.mark.parametrize("T,Hl,Wl,P", [(21, 30, 52, 8), (2, 5, 7, 3), (3, 8, 8, 8), (1, 9, 4, 4)])
def test_fractal_order_is_patch_bijection(T, Hl, Wl, P):
    n = T * Hl * Wl
    perm, st, ln, coords = ol.fractal_order(T, Hl, Wl, P, N=n + 5)
    assert sorted(perm.tolist()) == list(range(n + 5))
    assert (perm[n:] == np.arange(n, n + 5)).all()
    assert st[0] == 0 and (st[1:] == np.cumsum(ln)[:-1]).all() and ln.sum() == n
    xyz = token_coords(T, Hl, Wl)
    derived = ol.block_coords_from_tokens(xyz, perm, st, ln, P)
    assert (derived == coords).all()
    # time order kept, and raster order inside each patch
    assert (np.diff(xyz[perm[:n], 0]) >= 0).all()
    for s, m in zip(st, ln):
        assert (np.diff(perm[s:s + m]) > 0).all()
    # inverse permutation composes to the identity
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm))
    assert (perm[inv] == np.arange(len(perm))).all()


def test_fractal_patch_histogram_wan480():
    # 30 rows = 8+8+8+6 and 52 columns = 6*8+4 give, per frame, 18 patches of
    # 64 tokens, 6 of 48, 3 of 32 and 1 of 24.
    perm, st, ln, coords = ol.fractal_order(21, 30, 52, 8, N=32768)
    assert len(st) == 21 * 28
    vals, counts = np.unique(ln[:28], return_counts=True)
    assert dict(zip(vals.tolist(), counts.tolist())) == {24: 1, 32: 3, 48: 6, 64: 18}
    assert (ln.reshape(21, 28) == ln[:28]).all()


def _window_cases():
    with open(os.path.join(GOLDEN, "window_counts.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                g, tot, mx, mn = (s.strip() for s in line.split("|"))
                yield tuple(int(v) for v in g.split()), int(tot), int(mx), int(mn)


@pytest.mark.parametrize("grid,total,mx,mn", list(_window_cases()))
def test_window_counts_golden(grid, total, mx, mn):
    nt, ny, nx, rt, ry, rx = grid
    t, y, x = np.meshgrid(np.arange(nt), np.arange(ny), np.arange(nx), indexing="ij")
    c = np.stack([t.ravel(), y.ravel(), x.ravel()], 1)
    w = ol.window_blocks(c, c, rt, ry, rx)
    assert w.sum() == total and w.sum(1).max() == mx and w.sum(1).min() == mn
    assert (w == w.T).all() and w.diagonal().all()


def test_window_matches_token_level_brute_force():
    # Token pairs (i, j) are in the window iff their patches are; build it pair
    # by pair from coordinates and compare with the block window expanded.
    T, Hl, Wl, P = 3, 10, 9, 4
    perm, st, ln, coords = ol.fractal_order(T, Hl, Wl, P)
    w = ol.window_blocks(coords, coords, 1, 1, 1)
    xyz = token_coords(T, Hl, Wl)[perm]
    n = len(perm)
    blk = np.repeat(np.arange(len(st)), ln)
    for i in range(0, n, 7):
        for j in range(n):
            a, b = xyz[i], xyz[j]
            inside = (abs(a[0] - b[0]) <= 1 and abs(a[1] // P - b[1] // P) <= 1
                      and abs(a[2] // P - b[2] // P) <= 1)
            assert inside == w[blk[i], blk[j]]


# ----------------------------------------------------------- head-aware tiling

@pytest.mark.parametrize("T,Hl,Wl,P", [(21, 30, 52, 8), (2, 5, 7, 3), (3, 8, 8, 8)])
def test_tile_order_with_flat_boxes_is_the_fractal_order(T, Hl, Wl, P):
    a = ol.tile_order(T, Hl, Wl, 1, P, P, N=T * Hl * Wl + 3)
    b = ol.fractal_order(T, Hl, Wl, P, N=T * Hl * Wl + 3)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_tile_order_one_box_is_the_identity():
    perm, st, ln, co = ol.tile_order(3, 5, 7, 3, 5, 7)
    assert np.array_equal(perm, np.arange(105)) and st.tolist() == [0] and ln.tolist() == [105]
    assert co.tolist() == [[0, 0, 0]]


def _box_len(dim, p, b):
    return np.minimum(p, dim - b * p)


@pytest.mark.parametrize("T,Hl,Wl,pt,ph,pw", [(21, 30, 52, 2, 4, 8), (21, 30, 52, 4, 4, 4), (5, 6, 9, 2, 4, 8),
                                              (4, 7, 5, 3, 2, 5), (1, 3, 3, 4, 4, 4)])
def test_tile_order_blocks_are_boxes(T, Hl, Wl, pt, ph, pw):
    n = T * Hl * Wl
    perm, st, ln, co = ol.tile_order(T, Hl, Wl, pt, ph, pw, N=n + 4)
    assert sorted(perm.tolist()) == list(range(n + 4)) and (perm[n:] == np.arange(n, n + 4)).all()
    nbt, nby, nbx = -(-T // pt), -(-Hl // ph), -(-Wl // pw)
    assert len(st) == nbt * nby * nbx
    assert st[0] == 0 and (st[1:] == np.cumsum(ln)[:-1]).all() and ln.sum() == n
    # block b sits at grid position (bt, by, bx), row-major, frame boxes slowest
    g = np.arange(len(st))
    assert (co[:, 0] == g // (nby * nbx)).all() and (co[:, 1] == (g // nbx) % nby).all()
    assert (co[:, 2] == g % nbx).all()
    # closed-form box lengths (edge boxes are clipped)
    exp = _box_len(T, pt, co[:, 0]) * _box_len(Hl, ph, co[:, 1]) * _box_len(Wl, pw, co[:, 2])
    assert np.array_equal(ln, exp)
    xyz = token_coords(T, Hl, Wl)
    for b, (s, m) in enumerate(zip(st, ln)):
        c = xyz[perm[s:s + m]]
        assert (c // np.array([pt, ph, pw]) == co[b]).all()      # every token inside the box
        assert (np.diff(perm[s:s + m]) > 0).all()                 # raster order inside a box
