"""Pins of the reference block-sparse attention (no GPU)."""

import numpy as np
import torch

from oracle import attention as oa
from oracle import layout as ol
from oracle import mask as om


def _sdpa(q, k, v, mask=None):
    """torch's scaled_dot_product_attention in float64 on the CPU."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m)
    return o[0, 0].numpy()


def test_all_blocks_kept_is_dense_attention():
    rng = np.random.default_rng(10)
    n, d = 200, 32
    q, k, v = (rng.normal(size=(n, d)) for _ in range(3))
    st, ln = ol.raster_blocks(n, 64)
    keep, _ = om.block_mask(q, k, st, ln, st, ln, 0.0)
    o = oa.masked_attention(q, k, v, st, ln, st, ln, keep)
    np.testing.assert_allclose(o, _sdpa(q, k, v), rtol=0, atol=1e-12)


def test_window_only_mask_is_token_masked_attention():
    # Fractal blocks + a window-only block mask equals dense attention under a
    # token-level mask built from coordinates.
    T, Hl, Wl, P = 4, 9, 10, 4
    perm, st, ln, coords = ol.fractal_order(T, Hl, Wl, P)
    n = len(perm)
    rng = np.random.default_rng(11)
    q, k, v = (rng.normal(size=(n, 16)) for _ in range(3))
    keep = ol.window_blocks(coords, coords, 1, 1, 1)
    o = oa.permuted_attention(q, k, v, perm, perm, st, ln, st, ln, keep)
    from gen import token_coords
    xyz = token_coords(T, Hl, Wl)
    tile = np.stack([xyz[:, 0], xyz[:, 1] // P, xyz[:, 2] // P], 1)
    diff = np.abs(tile[:, None, :] - tile[None, :, :])
    tok = (diff[..., 0] <= 1) & (diff[..., 1] <= 1) & (diff[..., 2] <= 1)
    np.testing.assert_allclose(o, _sdpa(q, k, v, tok), rtol=0, atol=1e-12)


def test_two_keys_closed_form():
    rng = np.random.default_rng(12)
    q = rng.normal(size=(3, 4))
    k = rng.normal(size=(2, 4))
    v = rng.normal(size=(2, 4))
    st, ln = np.array([0, 1]), np.array([1, 1])
    o = oa.masked_attention(q[:2], k, v, st, ln, st, ln, np.ones((2, 2), bool), scale=0.5)
    s = 0.5 * q[:2] @ k.T
    a = 1.0 / (1.0 + np.exp(-(s[:, 0] - s[:, 1])))
    np.testing.assert_allclose(o, a[:, None] * v[0] + (1 - a)[:, None] * v[1], rtol=1e-13)


def test_sparse_rows_are_convex_combinations_and_blocks_respected():
    rng = np.random.default_rng(13)
    n, d = 256, 16
    q, k, v = (rng.normal(size=(n, d)) for _ in range(3))
    st, ln = ol.raster_blocks(n - 9, 64)
    keep = rng.random((len(st), len(st))) < 0.4
    keep[np.arange(len(st)), rng.integers(0, len(st), len(st))] = True
    o = oa.masked_attention(q, k, v, st, ln, st, ln, keep)
    assert (o[n - 9:] == 0).all()
    for I in range(len(st)):
        cols = np.concatenate([np.arange(st[J], st[J] + ln[J]) for J in np.nonzero(keep[I])[0]])
        rows = slice(st[I], st[I] + ln[I])
        assert (o[rows] >= v[cols].min(0) - 1e-12).all() and (o[rows] <= v[cols].max(0) + 1e-12).all()
        # the same rows from SDPA restricted to the kept columns
        np.testing.assert_allclose(o[rows], _sdpa(q[rows], k[cols], v[cols]), atol=1e-12)


def test_permutation_equivariance():
    rng = np.random.default_rng(14)
    n, d = 150, 8
    q, k, v = (rng.normal(size=(n, d)) for _ in range(3))
    pq = rng.permutation(n)
    pk = rng.permutation(n)
    qs, ql = np.array([0, 40, 90]), np.array([40, 50, 60])
    ks, kl = np.array([0, 30, 100]), np.array([30, 70, 50])
    keep = np.array([[1, 0, 1], [0, 1, 0], [1, 1, 1]], bool)
    o = oa.permuted_attention(q, k, v, pq, pk, qs, ql, ks, kl, keep)
    # token-level mask in the original order
    bq = np.empty(n, int)
    bk = np.empty(n, int)
    bq[pq] = np.repeat(np.arange(3), ql)
    bk[pk] = np.repeat(np.arange(3), kl)
    np.testing.assert_allclose(o, _sdpa(q, k, v, keep[bq][:, bk]), atol=1e-12)
