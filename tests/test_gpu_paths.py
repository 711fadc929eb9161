"""GPU parity of the reorder-based paths against the CPU reference (MI355X).

  * fractal flattening + CDF mask OR sliding-tile window + attention over
    variable-length patch blocks + inverse reorder (480p layer, 588 patches);
  * per-head box orders (head-aware tiling) + CDF mask + attention over each
    head's boxes + inverse reorder;
  * k-means of Q and K, cluster-contiguous order, centroid top-p mask,
    attention over variable-size cluster blocks, inverse permutation.

Integer work (permutations, cluster order, sizes) is compared bit-exactly.
Clusterings can differ from the reference's where distances nearly tie, so
k-means is checked by what must hold for any correct run (nearest-centroid
assignment w.r.t. the previous round's centroids, centroids equal to member
means, seeds drawn by the D^2 rule) and the later stages run on the GPU's own
clustering on both sides.
"""

import functools
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_avg_amd.pipelines as pl
from gen import WORKLOADS, generate, kmeans_uniforms, next_step, token_coords
from oracle import attention as oa
from oracle import kmeans as ok
from oracle import layout as ol
from oracle import mask as om
from tests.band import keep_from_lists, mask_mismatches

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=1)
def _wan480():
    w = WORKLOADS["wan480"]
    return generate(w)


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check_out(o_gpu, o_ref, rows, what):
    d = np.abs(o_gpu[rows] - o_ref[rows])
    say(f"  {what}: max-abs {d.max():.3e} mean-abs {d.mean():.3e}")
    assert np.isfinite(o_gpu[rows]).all(), what
    assert d.max() <= MAX_ABS and d.mean() <= MEAN_ABS, what


# ------------------------------------------------------------------ fractal + STA

def test_permute_roundtrip_bit_exact(gpu_lib):
    bsa = gpu_lib
    w = WORKLOADS["wan480_fractal_sta"]
    q, _, _ = _wan480()
    perm, st, ln, co = bsa.fractal_order(w.T, w.Hl, w.Wl, w.patch, w.N)
    rp, _, _, _ = ol.fractal_order(w.T, w.Hl, w.Wl, w.patch, w.N)
    assert np.array_equal(perm.numpy(), rp)
    qd = q.cuda()
    pd = perm.cuda()
    y = bsa.permute_tokens(qd, pd)
    assert torch.equal(y.cpu(), q[:, :, torch.from_numpy(rp)])
    assert torch.equal(bsa.unpermute_tokens(y, pd), qd)
    # per-head permutations
    rng = np.random.default_rng(3)
    ph = np.stack([rng.permutation(w.N) for _ in range(w.H)]).astype(np.int32)[None]
    y2 = bsa.permute_tokens(qd, torch.from_numpy(ph).cuda()).cpu()
    for h in (0, 7):
        assert torch.equal(y2[0, h], q[0, h][torch.from_numpy(ph[0, h]).long()])


def test_fractal_sta_path(gpu_lib):
    bsa = gpu_lib
    w = WORKLOADS["wan480_fractal_sta"]
    q, k, v = _wan480()
    say("fractal + STA path, 480p layer")
    lay = pl.fractal_layout(w.T, w.Hl, w.Wl, w.patch, w.N, "cuda")
    o, cnt, idx = pl.fractal_sta_attention(q.cuda(), k.cuda(), v.cuda(), lay, w.thr,
                                           radius=w.window, n_valid=w.n_valid, return_mask=True)
    torch.cuda.synchronize()
    assert gpu_lib.check_mask(cnt, idx, idx.shape[-1]) == (0, 0, 0)
    o, cnt, idx = _np(o), cnt.cpu().numpy(), idx.cpu().numpy()
    perm, st, ln, coords = ol.fractal_order(w.T, w.Hl, w.Wl, w.patch, w.N)
    derived = ol.block_coords_from_tokens(token_coords(w.T, w.Hl, w.Wl), perm, st, ln, w.patch)
    win = ol.window_blocks(derived, derived, *w.window)
    nb = len(st)
    assert (o[:, :, w.n_valid:] == 0).all()
    rng = np.random.default_rng(0)
    for h in (0, 5, 11):
        keep = keep_from_lists(cnt[0, h], idx[0, h], nb)
        qh, kh, vh = _np(q[0, h]), _np(k[0, h]), _np(v[0, h])
        ref_keep, P = om.block_mask(qh[perm], kh[perm], st, ln, st, ln, w.thr, window=win)
        assert (keep >= win).all(), "window bits must be set"
        bad = mask_mismatches(P, w.thr, keep, window=win)
        say(f"  head {h}: kept {keep.sum()}/{keep.size} (window alone {win.sum()}), "
            f"differing bits {(keep != ref_keep).sum()}, sure-bit mismatches {bad}")
        assert bad == 0
        blocks = sorted(set(rng.choice(nb, 12, replace=False).tolist()) | {0, nb - 1})
        ref = oa.permuted_attention(qh, kh, vh, perm, perm, st, ln, st, ln, keep, blocks=blocks)
        rows = perm[np.concatenate([np.arange(st[b], st[b] + ln[b]) for b in blocks])]
        _check_out(o[0, h], ref, rows, f"head {h} ({len(blocks)} patch blocks)")


def test_fractal_patch_tiles_match_gathered_keys(gpu_lib):
    # patches declared as at most 64 tokens run one tile per patch; the same
    # attention with undeclared lengths gathers key rows into 64-row chunks
    bsa = gpu_lib
    w = WORKLOADS["wan480_fractal_sta"]
    q, k, v = _wan480()
    heads = [0, 3]
    lay = pl.fractal_layout(w.T, w.Hl, w.Wl, w.patch, w.N, "cuda")
    assert lay.blocks.max_len == 64
    gat = bsa.Blocks(lay.blocks.start, lay.blocks.length)
    qp, kp, vp = (bsa.permute_tokens(t[:, heads].contiguous().cuda(), lay.perm) for t in (q, k, v))
    cnt, idx = bsa.build_block_mask(qp, kp, w.thr, window=(*lay.grid, *w.window), n_valid=w.n_valid,
                                    qb=lay.blocks, kb=lay.blocks)
    o1 = bsa.block_sparse_attn_fwd(qp, kp, vp, cnt, idx, n_valid=w.n_valid, qb=lay.blocks, kb=lay.blocks)
    o2 = bsa.block_sparse_attn_fwd(qp, kp, vp, cnt, idx, n_valid=w.n_valid, qb=gat, kb=gat)
    d = (o1.float() - o2.float()).abs()
    say(f"  patch tiles vs gathered keys: max-abs {float(d.max()):.3e} mean-abs {float(d.mean()):.3e}")
    assert float(d.max()) <= MAX_ABS and float(d.mean()) <= MEAN_ABS


def test_window_only_mask_is_static_sta(gpu_lib):
    # thr = 0 with the window keeps everything; with thr = 1 the kept set is
    # the window plus each row's heaviest block.
    bsa = gpu_lib
    w = WORKLOADS["wan480_fractal_sta"]
    q, k, v = _wan480()
    lay = pl.fractal_layout(w.T, w.Hl, w.Wl, w.patch, w.N, "cuda")
    qp = bsa.permute_tokens(q.cuda(), lay.perm)
    kp = bsa.permute_tokens(k.cuda(), lay.perm)
    cnt, idx = bsa.build_block_mask(qp, kp, 1.0, window=(*lay.grid, *w.window), n_valid=w.n_valid,
                                    qb=lay.blocks, kb=lay.blocks)
    cnt = cnt.cpu().numpy()
    perm, st, ln, coords = ol.fractal_order(w.T, w.Hl, w.Wl, w.patch, w.N)
    win = ol.window_blocks(coords, coords, *w.window)
    wc = win.sum(1)
    assert ((cnt[0] == wc[None]) | (cnt[0] == wc[None] + 1)).all()


# ------------------------------------------------------------------ head-aware tiling

def test_head_tiling_path(gpu_lib):
    # each head has its own box factorisation, so its own order and blocks
    # (588, 616 and 624 boxes, padded to 624 with empty blocks)
    bsa = gpu_lib
    w = WORKLOADS["wan480_head_tiling"]
    q, k, v = _wan480()
    factors = [w.tilings[h % len(w.tilings)] for h in range(w.H)]
    say(f"head-aware tiling path, 480p layer, factorisations {sorted(set(factors))}")
    lay = pl.head_tiling_layout(w.T, w.Hl, w.Wl, factors, w.N, w.B, "cuda")
    assert lay.nblocks[:3] == (588, 616, 624)
    o, cnt, idx = pl.head_tiled_attention(q.cuda(), k.cuda(), v.cuda(), lay, w.thr, n_valid=w.n_valid,
                                          return_mask=True)
    torch.cuda.synchronize()
    assert gpu_lib.check_mask(cnt, idx, idx.shape[-1]) == (0, 0, 0)
    o, cnt, idx = _np(o), cnt.cpu().numpy(), idx.cpu().numpy()
    assert (o[:, :, w.n_valid:] == 0).all()
    nbp = lay.blocks.nblocks
    rng = np.random.default_rng(1)
    for h in (0, 1, 2, 7):
        perm, st, ln, _ = ol.tile_order(w.T, w.Hl, w.Wl, *factors[h], w.N)
        assert np.array_equal(lay.perm[0, h].cpu().numpy(), perm)
        nb = len(st)
        stp = np.concatenate([st, np.full(nbp - nb, w.n_valid)])
        lnp = np.concatenate([ln, np.zeros(nbp - nb, np.int64)])
        keep = keep_from_lists(cnt[0, h], idx[0, h], nbp)
        assert not keep[nb:].any() and not keep[:, nb:].any(), "empty blocks take no part"
        keep = keep[:nb, :nb]
        qh, kh, vh = _np(q[0, h]), _np(k[0, h]), _np(v[0, h])
        ref_keep, P = om.block_mask(qh[perm], kh[perm], stp, lnp, stp, lnp, w.thr)
        assert not ref_keep[nb:].any() and not ref_keep[:, nb:].any()
        ref_keep, P = ref_keep[:nb, :nb], P[:nb, :nb]
        bad = mask_mismatches(P, w.thr, keep)
        say(f"  head {h} {factors[h]}: kept {keep.sum()}/{keep.size}, differing bits "
            f"{(keep != ref_keep).sum()}, sure-bit mismatches {bad}")
        assert bad == 0
        blocks = sorted(set(rng.choice(nb, 12, replace=False).tolist()) | {0, nb - 1})
        ref = oa.permuted_attention(qh, kh, vh, perm, perm, st, ln, st, ln, keep, blocks=blocks)
        rows = perm[np.concatenate([np.arange(st[b], st[b] + ln[b]) for b in blocks])]
        _check_out(o[0, h], ref, rows, f"head {h} ({len(blocks)} box blocks)")


# ------------------------------------------------------------------ semantic clustering

@functools.lru_cache(maxsize=1)
def _semantic():
    w = WORKLOADS["wan480_semantic"]
    q, k, v = _wan480()
    uq = torch.from_numpy(kmeans_uniforms(w.B, w.H, w.Cq, stream=0))
    uk = torch.from_numpy(kmeans_uniforms(w.B, w.H, w.Ck, stream=1))
    return w, q, k, v, uq, uk


def _d2(x, c):
    return ok.sq_dists(x, c)


def _check_seeding(xh, cent_h, uh, n):
    """Every seed is a token vector drawn by the D^2 inverse-CDF rule."""
    d2 = None
    for r in range(cent_h.shape[0]):
        hits = np.nonzero((xh == cent_h[r]).all(1))[0]
        assert len(hits) >= 1, r
        if r == 0:
            assert min(int(np.floor(uh[0] * n)), n - 1) in hits
            d2 = ((xh - cent_h[0]) ** 2).sum(1)
            continue
        cs = np.cumsum(d2)
        target = uh[r] * cs[-1]
        tol = 1e-5 * cs[-1]
        ok_idx = [i for i in hits if cs[i] - d2[i] <= target + tol and cs[i] >= target - tol]
        assert ok_idx, r
        d2 = np.minimum(d2, ((xh - cent_h[r]) ** 2).sum(1))


def _check_lloyd(xh, prev_h, cent_h, a_h, s_h):
    """The assignment is nearest w.r.t. the previous centroids (fp32 ties
    allowed), sizes count it, and centroids are their members' means."""
    C = cent_h.shape[0]
    assert np.array_equal(np.bincount(a_h, minlength=C), s_h)
    D = _d2(xh, prev_h)
    mine = D[np.arange(len(a_h)), a_h]
    assert (mine <= D.min(1) * (1 + 2e-5) + 1e-3).all()
    for c in range(C):
        if s_h[c]:
            ref = xh[a_h == c].mean(0)
            np.testing.assert_allclose(cent_h[c], ref, rtol=1e-5, atol=1e-4 * np.abs(ref).max())
        else:
            np.testing.assert_array_equal(cent_h[c], prev_h[c])


@pytest.mark.parametrize("which", ["q", "k"])
def test_kmeans_seeding_rule(gpu_lib, which):
    bsa = gpu_lib
    w, q, k, v, uq, uk = _semantic()
    x, C, u = (q, w.Cq, uq) if which == "q" else (k, w.Ck, uk)
    say(f"k-means++ seeding on {which}, C={C}")
    cent, a, sizes = bsa.kmeans(x.cuda(), C, 0, u.cuda(), n_valid=w.n_valid)
    cent = cent.cpu().numpy().astype(np.float64)
    for h in (0, 9):
        _check_seeding(_np(x[0, h])[:w.n_valid], cent[0, h], u[0, h].numpy().astype(np.float64), w.n_valid)


@pytest.mark.parametrize("d,C,n,N,H", [(64, 5, 650, 704, 2), (64, 40, 650, 704, 2), (128, 100, 1000, 1024, 1),
                                       (128, 1, 300, 320, 1), (64, 33, 2100, 2112, 3), (128, 37, 64, 64, 1),
                                       (64, 1024, 140000, 140032, 1)])
def test_kmeans_small_shapes(gpu_lib, d, C, n, N, H):
    """Head dims 64 and 128, cluster counts off the 32-centroid chunk of the
    assignment kernel, ragged token tails and a single cluster, and the
    supported maximum of 1024 clusters over 547 chunks of 256 tokens (the
    seeding draw holds 512 chunk sums in registers and reads the rest):
    the seeding rule, then four Lloyd rounds checked against the third's
    centroids."""
    bsa = gpu_lib
    g = torch.Generator().manual_seed(1000 + d + C + n)
    centres = torch.randn((H, 8, d), generator=g) * 3.0
    pick = torch.randint(0, 8, (H, N), generator=g)
    x = (torch.gather(centres, 1, pick[..., None].expand(H, N, d)) + torch.randn((H, N, d), generator=g))
    x[:, n:] = 0.0
    x = x[None].to(torch.bfloat16)
    u = torch.rand((1, H, C), generator=g, dtype=torch.float64).float()
    say(f"k-means d={d} C={C} n={n} N={N} H={H}")
    xd, ud = x.cuda(), u.cuda()
    seeds, _, _ = bsa.kmeans(xd, C, 0, ud, n_valid=n)
    c3, _, _ = bsa.kmeans(xd, C, 3, ud, n_valid=n)
    c4, a4, s4 = bsa.kmeans(xd, C, 4, ud, n_valid=n)
    torch.cuda.synchronize()
    seeds, c3, c4 = (t.cpu().numpy().astype(np.float64) for t in (seeds, c3, c4))
    a4, s4 = a4.cpu().numpy(), s4.cpu().numpy()
    assert (a4[:, :, n:] == -1).all()
    for h in range(H):
        xh = _np(x[0, h])[:n]
        _check_seeding(xh, seeds[0, h], u[0, h].numpy().astype(np.float64), n)
        _check_lloyd(xh, c3[0, h], c4[0, h], a4[0, h, :n], s4[0, h])


@pytest.mark.parametrize("which", ["q", "k"])
def test_kmeans_lloyd_invariants(gpu_lib, which):
    bsa = gpu_lib
    w, q, k, v, uq, uk = _semantic()
    x, C, u = (q, w.Cq, uq) if which == "q" else (k, w.Ck, uk)
    say(f"k-means Lloyd invariants on {which}, C={C}")
    xd, ud = x.cuda(), u.cuda()
    c9, a9, _ = bsa.kmeans(xd, C, w.kmeans_iters - 1, ud, n_valid=w.n_valid)
    c10, a10, s10 = bsa.kmeans(xd, C, w.kmeans_iters, ud, n_valid=w.n_valid)
    c10b, a10b, s10b = bsa.kmeans(xd, C, w.kmeans_iters, ud, n_valid=w.n_valid)
    assert torch.equal(c10, c10b) and torch.equal(a10, a10b), "k-means must be deterministic"
    c9, c10 = c9.cpu().numpy().astype(np.float64), c10.cpu().numpy().astype(np.float64)
    a10, s10 = a10.cpu().numpy(), s10.cpu().numpy()
    assert (a10[:, :, w.n_valid:] == -1).all()
    for h in (0, 4, 11):
        xh = _np(x[0, h])[:w.n_valid]
        ah = a10[0, h, :w.n_valid]
        assert np.array_equal(np.bincount(ah, minlength=C), s10[0, h])
        # the last assignment is nearest w.r.t. the previous centroids (fp32 ties allowed)
        D = _d2(xh, c9[0, h])
        mine = D[np.arange(len(ah)), ah]
        assert (mine <= D.min(1) * (1 + 2e-5) + 1e-3).all(), h
        # centroids are the means of their members (empty clusters keep their value)
        for c in range(C):
            if s10[0, h, c]:
                ref = xh[ah == c].mean(0)
                np.testing.assert_allclose(c10[0, h, c], ref, rtol=1e-5, atol=1e-4 * np.abs(ref).max())
        say(f"  head {h}: sizes min {s10[0, h].min()} max {s10[0, h].max()}, "
            f"inertia {((xh - c10[0, h][ah]) ** 2).sum():.6e}")


@pytest.mark.parametrize("which", ["q", "k"])
def test_kmeans_warm_start(gpu_lib, which):
    # centroids of one step start the clustering of the next (a drifted copy)
    bsa = gpu_lib
    w, q, k, v, uq, uk = _semantic()
    x, C, u = (q, w.Cq, uq) if which == "q" else (k, w.Ck, uk)
    x1 = next_step(x, 1, stream=0 if which == "q" else 1)
    say(f"k-means warm start on {which}, C={C}")
    xd, x1d, ud = x.cuda(), x1.cuda(), u.cuda()
    c0, _, _ = bsa.kmeans(xd, C, w.kmeans_iters, ud, n_valid=w.n_valid)
    cw, aw, sw, ch = bsa.kmeans_warm(x1d, c0, 40, n_valid=w.n_valid)
    cw2, aw2, sw2, ch2 = bsa.kmeans_warm(x1d, c0, 40, n_valid=w.n_valid)
    assert torch.equal(cw, cw2) and torch.equal(aw, aw2) and torch.equal(ch, ch2), "deterministic"
    ch = ch.cpu().numpy()
    assert (ch[..., 0] == w.n_valid).all()
    # once a round moves nothing, every later entry is 0
    for row in ch.reshape(-1, 40):
        z = np.nonzero(row == 0)[0]
        if len(z):
            assert (row[z[0]:] == 0).all()
    say(f"  moves per round, head 0: {ch[0, 0].tolist()}")
    # move counts: the assignments after t and t + 1 rounds differ in ch[t+1] tokens
    for t in (1, 2):
        _, a_t, _, _ = bsa.kmeans_warm(x1d, c0, t, n_valid=w.n_valid)
        _, a_t1, _, c_t1 = bsa.kmeans_warm(x1d, c0, t + 1, n_valid=w.n_valid)
        diff = (a_t != a_t1).sum(-1).cpu().numpy()
        assert np.array_equal(diff, c_t1.cpu().numpy()[..., t]), t
    # early exit is exact: a cold run of r rounds equals a warm start from its
    # seeds (which stops as soon as nothing moves), for r past convergence too
    seeds, _, _ = bsa.kmeans(xd, C, 0, ud, n_valid=w.n_valid)
    for r in (3, 25):
        cc, ac, sc = bsa.kmeans(xd, C, r, ud, n_valid=w.n_valid)
        cs, as_, ss, _ = bsa.kmeans_warm(xd, seeds, r, n_valid=w.n_valid)
        assert torch.equal(cc, cs) and torch.equal(ac, as_) and torch.equal(sc, ss), r
    # a move tolerance: each head stops after its first round with at most tol
    # moves, with the result of running exactly that many rounds
    tol = int(ch[0, :, 4].max())                 # every head gets there by round 4
    ct, at, _, cht = bsa.kmeans_warm(x1d, c0, 40, n_valid=w.n_valid, tol_moves=tol)
    cht = cht.cpu().numpy()[0]
    for h in (0, 5):
        row = cht[h]
        t_h = int(np.argmax(row <= tol))
        assert row[t_h] <= tol and (row[:t_h] > tol).all() and (row[t_h + 1:] == 0).all()
        cr, ar, _, _ = bsa.kmeans_warm(x1d, c0, t_h + 1, n_valid=w.n_valid)
        assert torch.equal(ct[0, h], cr[0, h]) and torch.equal(at[0, h], ar[0, h]), h
        say(f"  head {h}: tolerance {tol} moves reached after {t_h + 1} rounds")
    # round 0 against the oracle's assignment rule, from the same fp32 centroids
    c0n = c0.cpu().numpy().astype(np.float64)
    _, a1, _, _ = bsa.kmeans_warm(x1d, c0, 1, n_valid=w.n_valid)
    a1 = a1.cpu().numpy()
    cwn, aw_n, sw_n = cw.cpu().numpy().astype(np.float64), aw.cpu().numpy(), sw.cpu().numpy()
    for h in (0, 6):
        xh = _np(x1[0, h])[:w.n_valid]
        D = _d2(xh, c0n[0, h])
        ref = ok.assign(xh, c0n[0, h])
        mine = a1[0, h, :w.n_valid]
        gap = D[np.arange(len(mine)), mine] - D[np.arange(len(ref)), ref]
        bad = (mine != ref) & (gap > 2e-5 * D.min(1) + 1e-3)
        say(f"  head {h}: round-0 assignments differing from the oracle {(mine != ref).sum()}, "
            f"beyond fp32 ties {bad.sum()}")
        assert not bad.any()
        # the final centroids are the means of their members
        ah = aw_n[0, h, :w.n_valid]
        assert np.array_equal(np.bincount(ah, minlength=C), sw_n[0, h])
        for c in range(C):
            if sw_n[0, h, c]:
                r_ = xh[ah == c].mean(0)
                np.testing.assert_allclose(cwn[0, h, c], r_, rtol=1e-5, atol=1e-4 * np.abs(r_).max())


def test_semantic_path(gpu_lib):
    bsa = gpu_lib
    w, q, k, v, uq, uk = _semantic()
    say("semantic permutation path, 480p layer")
    o, st = pl.semantic_attention(q.cuda(), k.cuda(), v.cuda(), w.Cq, w.Ck, w.kmeans_iters, w.top_p,
                                  uq.cuda(), uk.cuda(), n_valid=w.n_valid, return_state=True)
    torch.cuda.synchronize()
    o = _np(o)
    assert (o[:, :, w.n_valid:] == 0).all()
    assert bsa.check_mask(st.kv_count, st.kv_index, w.Ck) == (0, 0, 0)
    cnt, idx = st.kv_count.cpu().numpy(), st.kv_index.cpu().numpy()
    cq, ck = st.cq.cpu().numpy(), st.ck.cpu().numpy()
    nq, nk = st.nq.cpu().numpy(), st.nk.cpu().numpy()
    pq, pk = st.perm_q.cpu().numpy(), st.perm_k.cpu().numpy()
    qs, ql = st.qblocks.start.cpu().numpy(), st.qblocks.length.cpu().numpy()
    ks, kl = st.kblocks.start.cpu().numpy(), st.kblocks.length.cpu().numpy()
    rng = np.random.default_rng(1)
    eff = tot = 0.0
    for h in (0, 6, 11):
        # cluster order: bit-exact stable sort of the GPU's own assignment
        aq = np.empty(w.n_valid, np.int64)
        ak = np.empty(w.n_valid, np.int64)
        for c in range(w.Cq):
            aq[pq[0, h, qs[0, h, c]:qs[0, h, c] + ql[0, h, c]]] = c
        for c in range(w.Ck):
            ak[pk[0, h, ks[0, h, c]:ks[0, h, c] + kl[0, h, c]]] = c
        rq, rqs, rql = ok.cluster_order(aq, w.Cq, w.N)
        rk, rks, rkl = ok.cluster_order(ak, w.Ck, w.N)
        assert np.array_equal(rq, pq[0, h]) and np.array_equal(rqs, qs[0, h]) and np.array_equal(rql, ql[0, h])
        assert np.array_equal(rk, pk[0, h]) and np.array_equal(rks, ks[0, h]) and np.array_equal(rkl, kl[0, h])
        assert np.array_equal(rql, nq[0, h]) and np.array_equal(rkl, nk[0, h])
        # centroid mask against the reference rule on the GPU's centroids
        keep = keep_from_lists(cnt[0, h], idx[0, h], w.Ck)
        ref_keep, W = om.centroid_mask(cq[0, h], nq[0, h], ck[0, h], nk[0, h], w.top_p)
        valid = nk[0, h] > 0
        rows = nq[0, h] > 0
        bad = mask_mismatches(W[rows][:, valid], 1.0 - w.top_p, keep[rows][:, valid])
        assert not keep[:, ~valid].any() and not keep[~rows].any()
        say(f"  head {h}: kept {keep.sum()}/{keep.size} cluster pairs, differing {(keep != ref_keep).sum()}, "
            f"sure-bit mismatches {bad}")
        assert bad == 0
        # attention over variable-size clusters, inverse-permuted
        qh, kh, vh = _np(q[0, h]), _np(k[0, h]), _np(v[0, h])
        blocks = sorted(rng.choice(np.nonzero(rows)[0], 6, replace=False).tolist())
        ref = oa.permuted_attention(qh, kh, vh, rq, rk, rqs, rql, rks, rkl, keep, blocks=blocks)
        rows_tok = rq[np.concatenate([np.arange(rqs[b], rqs[b] + rql[b]) for b in blocks])]
        _check_out(o[0, h], ref, rows_tok, f"head {h} ({len(blocks)} query clusters)")
        eff += float((rql[:, None] * rkl[None, :] * keep).sum())
        tot += float(w.n_valid) ** 2
    say(f"  kept token-pair density {eff / tot:.4f}")
