"""GPU parity of the mask-quality diagnostic (full-attention tile map and
mask recall) against the float64 CPU reference in oracle/diagnostic.py.

Tile statistics: relative 1e-3 (+1e-7 absolute): P comes from fp32 scores of
bf16 inputs and the forward's fp32 row normaliser. The recall's integer
decisions (which tiles make the equal-budget oracle mask) are taken on the
GPU's own fp32 tile maxima on both sides, so the oracle recall must match
exactly; the mass recall to 1e-5.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_avg_amd.pipelines as pl
from gen import WORKLOADS, generate
from oracle import diagnostic as od
from oracle import layout as ol
from tests.band import keep_from_lists

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check(q, k, cnt, idx, nv, heads):
    B, H, N, d = q.shape
    mq = pl.mask_quality(q.cuda(), k.cuda(), cnt.cuda(), idx.cuda(), n_valid=nv)
    mq2 = pl.mask_quality(q.cuda(), k.cuda(), cnt.cuda(), idx.cuda(), n_valid=nv)
    for a, b in ((mq.tile_max, mq2.tile_max), (mq.tile_sum, mq2.tile_sum), (mq.oracle_recall, mq2.oracle_recall)):
        assert torch.equal(a, b), "deterministic"
    st, ln = ol.raster_blocks(nv)
    nb = len(st)
    gmax, gsum, gmin = (_np(t)[0] for t in (mq.tile_max, mq.tile_sum, mq.tile_min))
    grec, gmass = _np(mq.oracle_recall)[0], _np(mq.mass_recall)[0]
    for h in heads:
        qh, kh = _np(q[0, h])[:nv], _np(k[0, h])[:nv]
        rmax, rsum, rmin = od.tile_stats(qh, kh, st, ln, st, ln)
        for g, r, what in ((gmax[h], rmax, "max"), (gsum[h], rsum, "sum"), (gmin[h], rmin, "min")):
            say(f"  head {h} tile {what}: max rel err {(np.abs(g - r) / np.maximum(np.abs(r), 1e-30)).max():.2e}")
            np.testing.assert_allclose(g, r, rtol=1e-3, atol=1e-7, err_msg=f"head {h} tile {what}")
        keep = keep_from_lists(cnt.numpy()[0, h], idx.numpy()[0, h], nb)
        rrec, rmass = od.mask_recall(keep, gmax[h], gsum[h])   # decisions on the GPU's fp32 maxima
        # same budget on both sides, so distinct recalls differ by >= 1/k >> 1e-6
        np.testing.assert_allclose(grec[h], rrec, rtol=0, atol=1e-6, err_msg=f"head {h} oracle recall")
        np.testing.assert_allclose(gmass[h], rmass, rtol=1e-5, atol=1e-7, err_msg=f"head {h} mass recall")
        # and against the oracle's own statistics: the mass recall to 1e-3
        _, rmass2 = od.mask_recall(keep, rmax, rsum)
        np.testing.assert_allclose(gmass[h], rmass2, rtol=1e-3, atol=1e-6)
        say(f"  head {h}: oracle recall {grec[h].mean():.4f}, mass recall {gmass[h].mean():.4f}")
    return mq


@pytest.mark.parametrize("H,N,nv,d", [(2, 704, 650, 128), (1, 320, 320, 64)])
def test_tile_stats_random_masks(gpu_lib, H, N, nv, d):
    say(f"tile statistics, random masks H={H} N={N} n_valid={nv} d={d}")
    rng = np.random.default_rng(N + d)
    x = (2.0 * rng.normal(size=(2, 1, H, N, d))).astype(np.float32)
    x[:, :, :, nv:] = 0
    q, k = (torch.from_numpy(x[i]).to(torch.bfloat16) for i in range(2))
    nb = -(-nv // 64)
    keep = rng.random((H, nb, nb)) < 0.4
    keep[:, 1, :] = False                          # a row that keeps nothing
    cnt = torch.from_numpy(keep.sum(2).astype(np.int32))[None]
    idx = torch.full((1, H, nb, nb), -1, dtype=torch.int32)
    for h in range(H):
        for i in range(nb):
            ids = np.nonzero(keep[h, i])[0]
            idx[0, h, i, :len(ids)] = torch.from_numpy(ids.astype(np.int32))
    mq = _check(q, k, cnt, idx, nv, range(H))
    assert (mq.oracle_recall[0, :, 1] == 0).all() and (mq.mass_recall[0, :, 1] == 0).all()


def test_tile_stats_mask_stage_lists(gpu_lib):
    # the mask stage's own lists on the first 4096 tokens of the 480p layer
    bsa = gpu_lib
    w = WORKLOADS["wan480"]
    q, k, _ = generate(w, heads=[0, 1])
    q, k = (t[:, :, :4096].contiguous() for t in (q, k))
    say("tile statistics on mask-stage lists, 480p layer, 4096 tokens")
    cnt, idx = bsa.build_block_mask(q.cuda(), k.cuda(), w.thr, n_valid=4096)
    _check(q, k, cnt.cpu(), idx.cpu(), 4096, [0, 1])


def test_tile_stats_wan480_full_layer_sampled(gpu_lib):
    # the whole 480p layer: sampled query-block rows of the tile map against
    # the oracle's full-attention rows, and their recall
    bsa = gpu_lib
    w = WORKLOADS["wan480"]
    q, k, _ = generate(w)
    nv = w.n_valid
    say("tile statistics, full 480p layer, sampled rows")
    cnt, idx = bsa.build_block_mask(q.cuda(), k.cuda(), w.thr, n_valid=nv)
    mq = pl.mask_quality(q.cuda(), k.cuda(), cnt, idx, n_valid=nv)
    torch.cuda.synchronize()
    gmax, gsum, gmin = (_np(t)[0] for t in (mq.tile_max, mq.tile_sum, mq.tile_min))
    grec, gmass = _np(mq.oracle_recall)[0], _np(mq.mass_recall)[0]
    cnt, idx = cnt.cpu().numpy()[0], idx.cpu().numpy()[0]
    st, ln = ol.raster_blocks(nv)
    nb = len(st)
    rng = np.random.default_rng(4)
    for h in (1, 10):
        kh = _np(k[0, h])[:nv]
        keep = keep_from_lists(cnt[h], idx[h], nb)
        for I in sorted(set(rng.choice(nb, 3, replace=False).tolist()) | {nb - 1}):
            qh = _np(q[0, h])[st[I]:st[I] + ln[I]]
            rmax, rsum, rmin = od.tile_stats(qh, kh, [0], [ln[I]], st, ln)
            for g, r, what in ((gmax[h, I], rmax[0], "max"), (gsum[h, I], rsum[0], "sum"),
                               (gmin[h, I], rmin[0], "min")):
                np.testing.assert_allclose(g, r, rtol=1e-3, atol=1e-7, err_msg=f"head {h} row {I} tile {what}")
            rrec, rmass = od.mask_recall(keep[I:I + 1], gmax[h, I:I + 1], gsum[h, I:I + 1])
            np.testing.assert_allclose(grec[h, I], rrec[0], rtol=0, atol=1e-6)
            np.testing.assert_allclose(gmass[h, I], rmass[0], rtol=1e-5, atol=1e-7)
            say(f"  head {h} row {I}: oracle recall {grec[h, I]:.3f} mass recall {gmass[h, I]:.3f}")


def test_mask_recall_max_key_blocks(gpu_lib):
    """The recall at the supported maximum of 8192 key blocks (the rows'
    maxima take 128 KiB of LDS per workgroup), on given tile maps: maxima
    with many exact ties (1000 distinct values, so the lower index decides),
    rows keeping nothing, one block, every block and random sets."""
    bsa = gpu_lib
    nq, nk = 40, 8192
    rng = np.random.default_rng(8192)
    tmax = (np.round(rng.random((nq, nk)) * 1000) / 1000).astype(np.float32)
    tsum = (rng.random((nq, nk)) * tmax).astype(np.float32)
    keep = rng.random((nq, nk)) < rng.choice([0.001, 0.01, 0.2, 0.5], size=(nq, 1))
    keep[0] = False
    keep[1] = True
    keep[2] = False
    keep[2, nk - 1] = True
    tsum[3] = 0.0                                    # a row with no attention mass
    cnt = keep.sum(1).astype(np.int32)
    idx = np.full((nq, nk), -1, np.int32)
    for i in range(nq):
        ids = np.flatnonzero(keep[i])
        idx[i, :len(ids)] = ids
    dev = lambda a: torch.from_numpy(a[None, None]).cuda()
    say(f"mask recall nqb={nq} nkb={nk}")
    rec, mass = bsa.mask_recall(dev(tmax), dev(tsum), dev(cnt), dev(idx))
    rec, mass = _np(rec)[0, 0], _np(mass)[0, 0]
    rrec, rmass = od.mask_recall(keep, tmax.astype(np.float64), tsum.astype(np.float64))
    say(f"  oracle recall {rrec.mean():.4f}, mass recall {rmass.mean():.4f}")
    np.testing.assert_allclose(rec, rrec, rtol=0, atol=1e-6)
    np.testing.assert_allclose(mass, rmass, rtol=1e-5, atol=1e-7)
    assert rec[0] == 0 and rec[1] == 1 and mass[1] == pytest.approx(1.0, abs=1e-6) and mass[3] == 0
