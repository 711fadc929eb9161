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


# ---------------------------------------------------------------- backward

def _token_mask(qstart, qlen, kstart, klen, keep, N):
    m = np.zeros((N, N), dtype=bool)
    for I in range(len(qstart)):
        for J in np.nonzero(keep[I])[0]:
            m[qstart[I]:qstart[I] + qlen[I], kstart[J]:kstart[J] + klen[J]] = True
    return m


def _autograd_masked(q, k, v, do, m, scale):
    # torch autograd of softmax(scale Q K^T + log mask) V in float64
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * qt @ kt.T
    s = s.masked_fill(~torch.tensor(m), float("-inf"))
    o = torch.softmax(s, dim=1) @ vt
    o.backward(torch.tensor(do, dtype=torch.float64))
    lse = torch.logsumexp(s.detach(), dim=1).numpy()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy(), lse


def _random_case(seed, N, d, nb):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.normal(size=(N, d)) for _ in range(4))
    st, ln = ol.raster_blocks(N, N // nb)
    keep = rng.random((len(st), len(st))) < 0.4
    keep[np.arange(len(st)), rng.integers(0, len(st), len(st))] = True    # every row keeps one
    return q, k, v, do, st, ln, keep


def test_backward_all_blocks_kept_is_dense_autograd():
    q, k, v, do, st, ln, _ = _random_case(1, 96, 8, 4)
    keep = np.ones((len(st), len(st)), bool)
    dq, dk, dv = oa.masked_attention_bwd(q, k, v, do, st, ln, st, ln, keep)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None])[0]
    o.backward(torch.tensor(do))
    for a, b in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        np.testing.assert_allclose(a, b.numpy(), rtol=1e-10, atol=1e-12)


def test_backward_and_lse_match_autograd_of_token_masked_softmax():
    q, k, v, do, st, ln, keep = _random_case(2, 120, 8, 5)
    scale = 0.37
    dq, dk, dv = oa.masked_attention_bwd(q, k, v, do, st, ln, st, ln, keep, scale=scale)
    lse = oa.masked_attention_lse(q, k, st, ln, st, ln, keep, scale=scale)
    rq, rk, rv, rl = _autograd_masked(q, k, v, do, _token_mask(st, ln, st, ln, keep, len(q)), scale)
    for a, b in ((dq, rq), (dk, rk), (dv, rv), (lse, rl)):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


def test_backward_finite_differences():
    # variable block lengths; loss = sum(O * do)
    rng = np.random.default_rng(3)
    N, d = 11, 3
    q, k, v, do = (rng.normal(size=(N, d)) for _ in range(4))
    st, ln = np.array([0, 4, 5]), np.array([4, 1, 6])
    keep = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], bool)
    dq, dk, dv = oa.masked_attention_bwd(q, k, v, do, st, ln, st, ln, keep)

    def loss(qq, kk, vv):
        return float((oa.masked_attention(qq, kk, vv, st, ln, st, ln, keep) * do).sum())

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for i, j in ((0, 0), (4, 2), (7, 1), (10, 0)):
            xp, xm = x.copy(), x.copy()
            xp[i, j] += h
            xm[i, j] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - g[i, j]) < 1e-6 * max(1.0, abs(fd)), (name, i, j, fd, g[i, j])


def test_backward_one_key_rows_closed_form():
    # every query block keeps a single one-token key block: P = 1, so the
    # scores get no gradient and dv is the upstream gradient summed per key
    rng = np.random.default_rng(4)
    N, d = 8, 4
    q, k, v, do = (rng.normal(size=(N, d)) for _ in range(4))
    qst, qln = np.array([0, 4]), np.array([4, 4])
    kst, kln = np.array([2, 6]), np.array([1, 1])
    keep = np.array([[1, 0], [0, 1]], bool)
    dq, dk, dv = oa.masked_attention_bwd(q, k, v, do, qst, qln, kst, kln, keep)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    ref = np.zeros_like(v)
    ref[2] = do[0:4].sum(0)
    ref[6] = do[4:8].sum(0)
    np.testing.assert_allclose(dv, ref, rtol=1e-14, atol=1e-14)
    lse = oa.masked_attention_lse(q, k, qst, qln, kst, kln, keep)
    np.testing.assert_allclose(lse[:4], q[:4] @ k[2] / 2.0, rtol=1e-14)
