"""GPU parity of the HIP path against the CPU reference (needs an MI355X).

Every case feeds the same seeded bf16 tensors to the library (through the C
ABI binding) and to the float64 reference, then compares:
  * pooled means: |gpu - ref| <= 1e-5 * mean|x| of the block (fp32 summation
    error bound for 64 terms is ~4e-6 of that);
  * masks: every bit the reference decides with margin (band.py: cumulative
    mass farther than 1e-4 from thr, near-ties within relative 1e-4 counted
    both ways) must match exactly, window bits must be set, lists ascending;
  * outputs: with the GPU's own mask, max-abs <= 2e-2 and mean-abs <= 2e-3
    against the float64 reference over valid rows;
  * integer work (permutations, counts): bit-exact.
"""

import functools
import sys

import numpy as np
import pytest
import torch

from gen import BY_INDEX, WORKLOADS, generate
from oracle import attention as oa
from oracle import layout as ol
from oracle import mask as om
from tests.band import keep_from_lists, mask_mismatches, set_violations

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=3)
def _inputs(key):
    w = WORKLOADS[key]
    q, k, v = generate(w)
    return w, q, k, v


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check_out(o_gpu, o_ref, rows, what):
    d = np.abs(o_gpu[rows] - o_ref[rows])
    say(f"  {what}: max-abs {d.max():.3e} mean-abs {d.mean():.3e}")
    assert np.isfinite(o_gpu[rows]).all(), what
    assert d.max() <= MAX_ABS and d.mean() <= MEAN_ABS, what


def _rows_of(st, ln, blocks):
    return np.concatenate([np.arange(st[b], st[b] + ln[b]) for b in blocks])


# --------------------------------------------------------------------- pooling

@pytest.mark.parametrize("key", ["tiny", "wan480"])
def test_pool_parity(gpu_lib, key):
    bsa = gpu_lib
    w, q, k, v = _inputs(key)
    say(f"pool parity {key}")
    qd = q.cuda()
    g = bsa.pool_blocks(qd, n_valid=w.n_valid).cpu().numpy()
    st, ln = ol.raster_blocks(w.n_valid)
    for h in range(min(w.H, 3)):
        x = _np(q[0, h])
        ref = om.pool(x, st, ln)
        scale = np.stack([np.abs(x[s:s + n]).mean(0) for s, n in zip(st, ln)])
        assert (np.abs(g[0, h] - ref) <= 1e-5 * scale + 1e-30).all(), h


def test_pool_descriptors_and_empty_blocks(gpu_lib):
    bsa = gpu_lib
    rng = np.random.default_rng(0)
    x = torch.from_numpy(rng.normal(size=(1, 2, 300, 64)).astype(np.float32)).to(torch.bfloat16)
    st = np.array([0, 10, 10, 77, 200], np.int32)
    ln = np.array([10, 0, 67, 100, 99], np.int32)
    blocks = bsa.Blocks(torch.from_numpy(st).cuda(), torch.from_numpy(ln).cuda())
    g = bsa.pool_blocks(x.cuda(), blocks=blocks).cpu().numpy()
    for h in range(2):
        ref = np.zeros((5, 64))
        for i in range(5):
            if ln[i]:
                ref[i] = om.pool(_np(x[0, h]), st[i:i + 1], ln[i:i + 1])[0]
        np.testing.assert_allclose(g[0, h], ref, rtol=1e-5, atol=1e-6)
        assert (g[0, h, 1] == 0).all()


# ------------------------------------------------------------------ mask stage

def _mask_case(bsa, w, q, k, heads, thr=None):
    thr = w.thr if thr is None else thr
    cnt, idx = bsa.build_block_mask(q.cuda(), k.cuda(), thr, n_valid=w.n_valid)
    cnt, idx = cnt.cpu().numpy(), idx.cpu().numpy()
    st, ln = ol.raster_blocks(w.n_valid)
    nb = len(st)
    total_bad = 0
    for h in heads:
        keep = keep_from_lists(cnt[0, h], idx[0, h], nb)
        ref_keep, P = om.block_mask(_np(q[0, h]), _np(k[0, h]), st, ln, st, ln, thr)
        bad = mask_mismatches(P, thr, keep)
        diff = int((keep != ref_keep).sum())
        say(f"  head {h}: kept {keep.sum()} / {keep.size}, differing bits {diff}, sure-bit mismatches {bad}")
        total_bad += bad
    return cnt, idx, total_bad


@pytest.mark.parametrize("key", ["tiny", "wan480"])
def test_mask_parity(gpu_lib, key):
    w, q, k, v = _inputs(key)
    say(f"mask parity {key}")
    heads = range(w.H) if key == "tiny" else [0, 3, 7, 11]
    _, _, bad = _mask_case(gpu_lib, w, q, k, heads)
    assert bad == 0


@pytest.mark.parametrize("thr", [0.0, 1.0, 0.5])
def test_mask_special_thresholds(gpu_lib, thr):
    w, q, k, v = _inputs("wan480")
    say(f"mask thr={thr}")
    cnt, idx, bad = _mask_case(gpu_lib, w, q, k, [1], thr=thr)
    assert bad == 0
    if thr == 0.0:
        assert (cnt == w.nb).all()
    if thr == 1.0:
        assert (cnt >= 1).all() and (cnt <= 2).all()


def test_mask_ragged_and_d64(gpu_lib):
    bsa = gpu_lib
    rng = np.random.default_rng(1)
    for (H, N, nv, d, g) in [(3, 640, 600, 64, 4.0), (2, 1280, 1250, 128, 3.0)]:
        say(f"mask ragged H={H} N={N} n_valid={nv} d={d}")
        x = rng.normal(size=(2, 1, H, N, d)).astype(np.float32) * g
        x[:, :, :, nv:] = 0
        q = torch.from_numpy(x[0]).to(torch.bfloat16)
        k = torch.from_numpy(x[1]).to(torch.bfloat16)
        cnt, idx = bsa.build_block_mask(q.cuda(), k.cuda(), 0.15, n_valid=nv)
        cnt, idx = cnt.cpu().numpy(), idx.cpu().numpy()
        st, ln = ol.raster_blocks(nv)
        for h in range(H):
            keep = keep_from_lists(cnt[0, h], idx[0, h], len(st))
            _, P = om.block_mask(_np(q[0, h]), _np(k[0, h]), st, ln, st, ln, 0.15)
            assert mask_mismatches(P, 0.15, keep) == 0


def test_mask_deterministic(gpu_lib):
    w, q, k, v = _inputs("wan480")
    qd, kd = q.cuda(), k.cuda()
    a = gpu_lib.build_block_mask(qd, kd, w.thr, n_valid=w.n_valid)
    b = gpu_lib.build_block_mask(qd, kd, w.thr, n_valid=w.n_valid)
    assert torch.equal(a[0], b[0])
    for r in range(0, a[0].numel(), 97):
        c = int(a[0].view(-1)[r])
        assert torch.equal(a[1].view(-1, a[1].shape[-1])[r, :c], b[1].view(-1, b[1].shape[-1])[r, :c])


def _list_defects(cnt, idx, nkb):
    """Host count of what bsa_check_mask reports, from its definition."""
    cnt = cnt.reshape(-1)
    idx = idx.reshape(len(cnt), -1)
    stride = idx.shape[1]
    bad_rows = oor = uns = 0
    for r, c in enumerate(cnt):
        if c < 0 or c > stride:
            bad_rows += 1
            continue
        row = idx[r, :c]
        oor += int(((row < 0) | (row >= nkb)).sum())
        uns += int((row[1:] <= row[:-1]).sum())
    return bad_rows, oor, uns


def test_check_mask_counts_defects(gpu_lib):
    """The list validator finds nothing in the mask stage's lists and counts
    planted defects exactly: counts outside [0, stride], ids outside
    [0, nkb), entries out of ascending order (a swap, a repeat)."""
    bsa = gpu_lib
    w, q, k, v = _inputs("wan480")
    cnt, idx = bsa.build_block_mask(q.cuda(), k.cuda(), w.thr, n_valid=w.n_valid)
    nkb = (w.n_valid + 63) // 64
    say(f"check_mask on the 480p lists ({cnt.numel()} rows)")
    assert bsa.check_mask(cnt, idx, nkb) == (0, 0, 0)
    c, x = cnt.cpu().numpy().copy(), idx.cpu().numpy().copy()
    flat_c, flat_x = c.reshape(-1), x.reshape(len(c.reshape(-1)), -1)
    long_rows = np.nonzero(flat_c >= 4)[0]
    flat_c[3] = -1
    flat_c[5] = flat_x.shape[1] + 1
    r = long_rows[10]
    flat_x[r, 1] = nkb                                # out of range (and not ascending after it)
    r = long_rows[20]
    flat_x[r, [1, 2]] = flat_x[r, [2, 1]]             # swapped pair
    r = long_rows[30]
    flat_x[r, 2] = flat_x[r, 1]                       # repeated id
    r = long_rows[40]
    flat_x[r, 0] = -7
    want = _list_defects(c, x, nkb)
    got = bsa.check_mask(torch.from_numpy(c).cuda(), torch.from_numpy(x).cuda(), nkb)
    say(f"  planted defects: expected {want}, counted {got}")
    assert want[0] == 2 and want[1] == 2 and want[2] >= 3
    assert got == want


def test_mask_exact_ties(gpu_lib):
    """All scores equal: the cut falls inside one run of ties.

    Every block has the same mass 1/n, so dropping lightest-first with the
    higher index lighter drops the top indices while the inclusive sum stays
    below thr: with n = 600 and thr = 0.5004 exactly 300 blocks go and every
    row keeps J = 0..299 (300/600 < 0.5004 < 301/600). Exercises the path
    where more than 64 keys share the leading radix digits.
    """
    n, d = 600, 64
    x = torch.full((1, 1, n * 64, d), 0.5, dtype=torch.bfloat16)
    cnt, idx = gpu_lib.build_block_mask(x.cuda(), x.cuda(), 0.5004)
    cnt, idx = cnt.cpu().numpy(), idx.cpu().numpy()
    ref = om.cdf_keep(np.full(n, 1.0 / n), 0.5004)
    assert ref.sum() == 300 and ref[:300].all()
    assert (cnt == 300).all()
    assert (idx[0, 0, :, :300] == np.arange(300)).all()
    keep = keep_from_lists(cnt[0, 0], idx[0, 0], n)
    assert all(set_violations(np.full(n, 1.0 / n), 0.5004, row) == 0 for row in keep)


@pytest.mark.parametrize("nkb", [1000, 2112])
def test_mask_long_rows(gpu_lib, nkb):
    """Row lengths beyond the 512-block workloads: 1000 key blocks (16
    elements per lane) and 2112 (rows streamed from LDS)."""
    rng = np.random.default_rng(nkb)
    N, d = nkb * 64, 64
    ph = rng.normal(size=(N, 8)) @ rng.normal(size=(8, d)) * 0.7
    x = (ph[None, None] + 0.3 * rng.normal(size=(2, 1, N, d))).astype(np.float32)
    q = torch.from_numpy(x[0:1, 0:1].reshape(1, 1, N, d)).to(torch.bfloat16)
    k = torch.from_numpy(x[1:2, 0:1].reshape(1, 1, N, d)).to(torch.bfloat16)
    say(f"mask long rows nkb={nkb}")
    cnt, idx = gpu_lib.build_block_mask(q.cuda(), k.cuda(), 0.2)
    cnt, idx = cnt.cpu().numpy(), idx.cpu().numpy()
    st, ln = ol.raster_blocks(N)
    keep = keep_from_lists(cnt[0, 0], idx[0, 0], nkb)
    rows = np.arange(0, nkb, 7)
    _, P = om.block_mask(_np(q[0, 0]), _np(k[0, 0]), st, ln, st, ln, 0.2)
    bad = mask_mismatches(P[rows], 0.2, keep[rows])
    say(f"  kept {keep[rows].sum()} of {keep[rows].size}, sure-bit mismatches {bad}")
    assert bad == 0
    assert (cnt >= 1).all()


@pytest.mark.parametrize("nkb,d,H,nv_cut,win", [(1025, 128, 3, 0, None), (1500, 64, 2, 37, None),
                                                   (2048, 128, 2, 0, None), (1200, 128, 2, 20, (3, 20, 20, 1, 2, 2))])
def test_mask_rows_1025_to_2048(gpu_lib, nkb, d, H, nv_cut, win):
    """Rows of 1025..2048 key blocks (the 720p layer's class; at d = 128 the
    pipelined kernel with split bf16 scores): both head dims, several heads,
    a ragged last block, row counts that are not a multiple of 16, the
    2048-block edge where the score rows and histograms fill the LDS, the
    window union, and the fused call against pooling and selecting in two
    calls."""
    rng = np.random.default_rng(nkb + d)
    nv = nkb * 64 - nv_cut
    N = nkb * 64
    ph = rng.normal(size=(N, 8)) @ rng.normal(size=(8, d)) * 0.7
    x = (ph[None, None] + 0.3 * rng.normal(size=(2, H, N, d))).astype(np.float32)
    x[:, :, nv:] = 0
    q = torch.from_numpy(x[0][None]).to(torch.bfloat16)
    k = torch.from_numpy(x[1][None]).to(torch.bfloat16)
    say(f"mask rows nkb={nkb} d={d} H={H} n_valid={nv} window={win}")
    cnt, idx = gpu_lib.build_block_mask(q.cuda(), k.cuda(), 0.2, window=win, n_valid=nv)
    cnt, idx = cnt.cpu().numpy(), idx.cpu().numpy()
    # pooling and selecting in two calls gives the same lists as the fused call
    qbar = gpu_lib.pool_blocks(q.cuda(), n_valid=nv)
    kbar = gpu_lib.pool_blocks(k.cuda(), n_valid=nv)
    cnt2, idx2 = gpu_lib.select_blocks(qbar, kbar, 0.2, window=win)
    cnt2, idx2 = cnt2.cpu().numpy(), idx2.cpu().numpy()
    assert np.array_equal(cnt2, cnt)
    for h in range(H):
        assert np.array_equal(keep_from_lists(cnt2[0, h], idx2[0, h], nkb), keep_from_lists(cnt[0, h], idx[0, h], nkb))
    st, ln = ol.raster_blocks(nv)
    assert len(st) == nkb
    W = None
    if win is not None:
        nt, ny, nx = win[:3]
        J = np.arange(nkb)
        coords = np.stack([J // (nx * ny), (J // nx) % ny, J % nx], axis=1)
        W = ol.window_blocks(coords, coords, *win[3:])
    total = 0
    for h in range(H):
        keep = keep_from_lists(cnt[0, h], idx[0, h], nkb)
        rows = np.unique(np.concatenate([np.arange(h, nkb, 23), np.arange(nkb - 9, nkb)]))
        _, P = om.block_mask(_np(q[0, h]), _np(k[0, h]), st, ln, st, ln, 0.2)
        bad = mask_mismatches(P[rows], 0.2, keep[rows], window=None if W is None else W[rows])
        if W is not None:
            assert (keep >= W).all(), "window bits must be set"
        say(f"  head {h}: kept {keep[rows].sum()} of {keep[rows].size}, mismatches {bad}")
        total += bad
    assert total == 0
    assert (cnt >= 1).all()



@pytest.mark.parametrize("nkb,d", [(3000, 128), (8192, 64), (8192, 128)])
def test_mask_max_key_blocks(gpu_lib, nkb, d):
    """Rows past 2048 key blocks, where the scores are streamed from LDS:
    2049..4096 at d = 128 (eight rows per workgroup) and the supported
    maximum of 8192 key blocks (four rows per workgroup; the block index of
    the radix key reaches its last 13-bit value), with a ragged last block.
    Inputs are smooth within each 64-token block (a per-block latent plus
    token noise), which keeps ~8-24 % of the blocks at thr = 0.2. Sampled
    rows against the reference's block probabilities (pooling, scores and
    row softmax for those rows only: rows are independent)."""
    rng = np.random.default_rng(nkb + d)
    N = nkb * 64
    nv = N - 29
    zb = rng.normal(size=(nkb, 8)).astype(np.float32)
    W = rng.normal(size=(8, d)).astype(np.float32) * 0.25
    qb_ = np.repeat(zb @ W, 64, axis=0)
    kb_ = np.repeat((zb + 0.5 * rng.normal(size=(nkb, 8)).astype(np.float32)) @ W, 64, axis=0)
    q = torch.from_numpy((qb_ + 0.3 * rng.normal(size=(N, d)).astype(np.float32))[None, None]).to(torch.bfloat16)
    k = torch.from_numpy((kb_ + 0.3 * rng.normal(size=(N, d)).astype(np.float32))[None, None]).to(torch.bfloat16)
    del qb_, kb_
    q[:, :, nv:] = 0
    k[:, :, nv:] = 0
    say(f"mask max key blocks nkb={nkb} d={d} n_valid={nv}")
    cnt, idx = gpu_lib.build_block_mask(q.cuda(), k.cuda(), 0.2, n_valid=nv)
    cnt, idx = cnt.cpu().numpy(), idx.cpu().numpy()
    st, ln = ol.raster_blocks(nv)
    assert len(st) == nkb and ln[-1] == 64 - 29
    rows = np.unique(np.concatenate([np.arange(0, nkb, 61), np.arange(nkb - 5, nkb)]))
    keep = keep_from_lists(cnt[0, 0][rows], idx[0, 0][rows], nkb)
    qbar = om.pool(_np(q[0, 0]), st, ln)
    kbar = om.pool(_np(k[0, 0]), st, ln)
    P = om.softmax_rows(om.reduced_scores(qbar[rows], kbar, 1.0 / np.sqrt(d)))
    bad = mask_mismatches(P, 0.2, keep)
    say(f"  kept {keep.sum()} of {keep.size} over {len(rows)} rows, mismatches {bad}")
    assert bad == 0
    assert (cnt >= 1).all() and (cnt <= nkb).all()

# ------------------------------------------------------------------- attention

def _attn_case(bsa, w, q, k, v, heads, nsample, seed=0, thr=None):
    thr = w.thr if thr is None else thr
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    cnt, idx = bsa.build_block_mask(qd, kd, thr, n_valid=w.n_valid)
    o = bsa.block_sparse_attn_fwd(qd, kd, vd, cnt, idx, n_valid=w.n_valid)
    torch.cuda.synchronize()
    o = _np(o)
    cnt, idx = cnt.cpu().numpy(), idx.cpu().numpy()
    st, ln = ol.raster_blocks(w.n_valid)
    nb = len(st)
    rng = np.random.default_rng(seed)
    for h in heads:
        keep = keep_from_lists(cnt[0, h], idx[0, h], nb)
        blocks = list(range(nb)) if nsample is None else sorted(
            set(rng.choice(nb, size=min(nsample, nb), replace=False).tolist()) | {0, nb - 1})
        ref = oa.masked_attention(_np(q[0, h]), _np(k[0, h]), _np(v[0, h]), st, ln, st, ln, keep,
                                  blocks=blocks)
        rows = _rows_of(st, ln, blocks)
        _check_out(o[0, h], ref, rows, f"head {h} ({len(blocks)} query blocks)")
    assert (o[:, :, w.n_valid:] == 0).all()
    return o


def test_attn_parity_tiny(gpu_lib):
    w, q, k, v = _inputs("tiny")
    say("attention parity tiny (every block)")
    _attn_case(gpu_lib, w, q, k, v, range(w.H), None)


def test_attn_parity_wan480(gpu_lib):
    w, q, k, v = _inputs("wan480")
    say("attention parity wan480 (sampled query blocks)")
    _attn_case(gpu_lib, w, q, k, v, [0, 5, 11], 10)


def test_attn_parity_wan480_every_block_one_head(gpu_lib):
    w, q, k, v = _inputs("wan480")
    say("attention parity wan480 head 6, every query block")
    _attn_case(gpu_lib, w, q, k, v, [6], None)


def test_attn_dense_equivalence(gpu_lib):
    # thr = 0 keeps every block: the result is dense softmax attention.
    w, q, k, v = _inputs("tiny")
    say("attention thr=0 == dense")
    o = _attn_case(gpu_lib, w, q, k, v, range(w.H), None, thr=0.0)
    for h in range(w.H):
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[0, h].double()[None], k[0, h].double()[None], v[0, h].double()[None])[0].numpy()
        _check_out(o[0, h], ref, np.arange(w.n_valid), f"dense head {h}")


@pytest.mark.parametrize("H,N,nv,d", [(2, 256, 256, 64), (3, 704, 650, 128), (1, 1088, 1030, 64)])
def test_attn_ragged_random_masks(gpu_lib, H, N, nv, d):
    # random kept lists (including long and single-block rows) on ragged sizes
    bsa = gpu_lib
    say(f"attention random masks H={H} N={N} n_valid={nv} d={d}")
    rng = np.random.default_rng(N)
    x = rng.normal(size=(3, 1, H, N, d)).astype(np.float32)
    x[:, :, :, nv:] = 0
    q, k, v = (torch.from_numpy(x[i] * (2.0 if i < 2 else 1.0)).to(torch.bfloat16) for i in range(3))
    st, ln = ol.raster_blocks(nv)
    nb = len(st)
    keep = rng.random((H, nb, nb)) < 0.3
    keep[:, :, 0] |= ~keep.any(2)
    keep[:, 0, :] = True
    cnt = keep.sum(2).astype(np.int32)
    idx = np.full((H, nb, nb), -1, np.int32)
    for h in range(H):
        for i in range(nb):
            ids = np.nonzero(keep[h, i])[0]
            idx[h, i, :len(ids)] = ids
    o = bsa.block_sparse_attn_fwd(q.cuda(), k.cuda(), v.cuda(), torch.from_numpy(cnt[None]).cuda(),
                                  torch.from_numpy(idx[None]).cuda(), n_valid=nv)
    o = _np(o)
    for h in range(H):
        ref = oa.masked_attention(_np(q[0, h]), _np(k[0, h]), _np(v[0, h]), st, ln, st, ln, keep[h])
        _check_out(o[0, h], ref, np.arange(nv), f"head {h}")
    assert (o[:, :, nv:] == 0).all()


def test_attn_empty_rows_give_zero(gpu_lib):
    bsa = gpu_lib
    q = torch.randn(1, 1, 128, 64, dtype=torch.bfloat16)
    cnt = torch.tensor([[[0, 1]]], dtype=torch.int32)
    idx = torch.tensor([[[[0, -1], [1, -1]]]], dtype=torch.int32)
    o = bsa.block_sparse_attn_fwd(q.cuda(), q.cuda(), q.cuda(), cnt.cuda(), idx.cuda()).cpu()
    assert (o[0, 0, :64] == 0).all() and o[0, 0, 64:].abs().sum() > 0


def test_attn_pad_poisoning_and_determinism(gpu_lib):
    bsa = gpu_lib
    w, q, k, v = _inputs("wan480")
    say("pad poisoning + determinism wan480")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    cnt, idx = bsa.build_block_mask(qd, kd, w.thr, n_valid=w.n_valid)
    o1 = bsa.block_sparse_attn_fwd(qd, kd, vd, cnt, idx, n_valid=w.n_valid)
    for rep in range(5):
        o2 = bsa.block_sparse_attn_fwd(qd, kd, vd, cnt, idx, n_valid=w.n_valid)
        assert torch.equal(o1, o2), rep
    for val in (float("nan"), 1e4):
        qp, kp, vp = qd.clone(), kd.clone(), vd.clone()
        for t in (qp, kp, vp):
            t[:, :, w.n_valid:] = val
        c2, i2 = bsa.build_block_mask(qp, kp, w.thr, n_valid=w.n_valid)
        assert torch.equal(c2, cnt)
        o3 = bsa.block_sparse_attn_fwd(qp, kp, vp, c2, i2, n_valid=w.n_valid)
        assert torch.equal(o3, o1), val


# ---------------------------------------------------------------- full-size 720p

@pytest.mark.parametrize("part", ["mask", "attn"])
def test_hunyuan720_sampled(gpu_lib, part):
    w, q, k, v = _inputs("hunyuan720")
    say(f"hunyuan720 {part} (sampled heads / blocks)")
    if part == "mask":
        _, _, bad = _mask_case(gpu_lib, w, q, k, [0, 23])
        assert bad == 0
    else:
        _attn_case(gpu_lib, w, q, k, v, [4, 19], 5)


@pytest.mark.parametrize("path", ["split", "one_wave"])
def test_attn_long_rows(gpu_lib, path):
    # >= 1024 uniform key blocks at d = 128: with the full workspace the rows
    # run split over key segments (plan, items, partials merged by each query
    # block's last item); with only the order table the one-wave kernel runs
    # them whole. Random kept lists
    # (a dense row, rows inside one segment, a row keeping nothing, the
    # ragged last block) on a ragged length, sampled query blocks (and their
    # log-normalisers) against the oracle, then repeat runs and poisoned
    # padding must give the same bits
    bsa = gpu_lib
    H, d, nkb = 2, 128, 1025
    N = nkb * 64
    nv = N - 37
    say(f"attention long rows ({path}) H={H} N={N} n_valid={nv}")
    rng = np.random.default_rng(1025)
    x = rng.normal(size=(3, 1, H, N, d)).astype(np.float32)
    x[:, :, :, nv:] = 0
    q, k, v = (torch.from_numpy(x[i] * (2.0 if i < 2 else 1.0)).to(torch.bfloat16) for i in range(3))
    st, ln = ol.raster_blocks(nv)
    assert len(st) == nkb
    keep = rng.random((H, nkb, nkb)) < 0.03
    keep[:, :, nkb - 1] |= rng.random((H, nkb)) < 0.3       # ragged last key block
    keep[:, :, 0] |= ~keep.any(2)
    keep[:, 5, :] = True                                     # one dense row
    keep[:, 9, :] = False
    keep[:, 9, 700] = True                                   # one single-block row
    keep[:, 10, :] = False
    keep[:, 10, 260:300] = True                              # a row inside one key segment
    keep[:, 11, :] = False                                   # a row keeping nothing
    keep[:, nkb - 1, :] = False
    keep[:, nkb - 1, [3, 255, 256, 511, 512, 1024]] = True   # segment edges, ragged last query block
    cnt = keep.sum(2).astype(np.int32)
    idx = np.full((H, nkb, nkb), -1, np.int32)
    for h in range(H):
        for i in range(nkb):
            ids = np.nonzero(keep[h, i])[0]
            idx[h, i, :len(ids)] = ids
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    cd, id_ = torch.from_numpy(cnt[None]).cuda(), torch.from_numpy(idx[None]).cuda()
    lib = bsa.load()
    full = lib.bsa_block_sparse_attn_fwd_workspace(1, H, nkb, None)
    small = (4 * H * (nkb + 1) + 255) // 256 * 256
    assert full > small
    ws = torch.empty(full if path == "split" else small, dtype=torch.uint8, device="cuda")
    o1, lse = bsa.block_sparse_attn_fwd_lse(qd, kd, vd, cd, id_, n_valid=nv, workspace=ws)
    o = _np(o1)
    lse = lse.cpu().numpy()
    blocks = sorted({0, 5, 9, 10, 11, nkb - 1} | set(rng.choice(nkb, 10, replace=False).tolist()))
    for h in range(H):
        args = (_np(q[0, h]), _np(k[0, h]))
        ref = oa.masked_attention(*args, _np(v[0, h]), st, ln, st, ln, keep[h], blocks=blocks)
        _check_out(o[0, h], ref, _rows_of(st, ln, blocks), f"head {h} ({len(blocks)} query blocks)")
        ref_lse = oa.masked_attention_lse(*args, st, ln, st, ln, keep[h])
        rows = _rows_of(st, ln, blocks)
        fin = np.isfinite(ref_lse[rows])
        assert np.array_equal(fin, np.isfinite(lse[0, h, rows]))
        # the one-wave kernel sums the bf16-rounded P that PV multiplies (so O
        # is a convex combination with exactly those weights): its row sum is
        # within a relative 2^-8 of the exact one, its log within 4e-3
        tol = 1e-3 if path == "split" else 4e-3
        assert np.abs(lse[0, h, rows][fin] - ref_lse[rows][fin]).max() <= tol
    assert (o[:, :, nv:] == 0).all()
    assert (o[:, :, st[11]:st[11] + 64] == 0).all()          # no kept block: zero rows
    assert np.isneginf(lse[:, :, nv:]).all()
    o2 = bsa.block_sparse_attn_fwd(qd, kd, vd, cd, id_, n_valid=nv, workspace=ws)
    assert torch.equal(o1, o2)
    for t in (qd, kd, vd):
        t[:, :, nv:] = float("nan")
    o3 = bsa.block_sparse_attn_fwd(qd, kd, vd, cd, id_, n_valid=nv, workspace=ws)
    assert torch.equal(o1, o3)


@pytest.mark.parametrize("d", [64, 128])
def test_attn_max_key_blocks(gpu_lib, d):
    """The supported maximum of 8192 query and key blocks. At d = 128 the
    split plan's bucket counts do not fit its LDS there, and at either head
    dim the longest-first order table is one word past its 64 KiB, so the
    rows run whole on the two-wave kernel in block order, with the pad rows
    zeroed by a launch of their own. Random lists with a dense row (8192
    chunks), a single-block row, a row keeping nothing and the ragged last
    block; sampled query blocks against the reference, then a repeat run
    and poisoned padding must give the same bits."""
    bsa = gpu_lib
    nkb = 8192
    N = nkb * 64
    nv = N - 37
    rng = np.random.default_rng(8192 + d)
    say(f"attention max key blocks d={d} N={N} n_valid={nv}")
    x = [rng.normal(size=(N, d)).astype(np.float32) for _ in range(3)]
    for t in x:
        t[nv:] = 0
    q, k, v = (torch.from_numpy(t[None, None] * (2.0 if i < 2 else 1.0)).to(torch.bfloat16)
               for i, t in enumerate(x))
    del x
    st, ln = ol.raster_blocks(nv)
    assert len(st) == nkb
    keep = rng.random((nkb, nkb), dtype=np.float32) < 0.01
    keep[:, nkb - 1] |= rng.random(nkb, dtype=np.float32) < 0.2     # ragged last key block
    keep[:, 0] |= ~keep.any(1)
    keep[5, :] = True                                                # a dense row
    keep[9, :] = False
    keep[9, 4097] = True                                             # a single-block row
    keep[11, :] = False                                              # a row keeping nothing
    keep[nkb - 1, :] = False
    keep[nkb - 1, [0, 383, 384, 4095, 4096, nkb - 1]] = True          # ragged last query block
    cnt = keep.sum(1).astype(np.int32)
    idx = np.full((nkb, nkb), -1, np.int32)
    for i in range(nkb):
        ids = np.flatnonzero(keep[i])
        idx[i, :len(ids)] = ids
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    cd, id_ = torch.from_numpy(cnt[None, None]).cuda(), torch.from_numpy(idx[None, None]).cuda()
    del idx
    o1 = bsa.block_sparse_attn_fwd(qd, kd, vd, cd, id_, n_valid=nv)
    o = _np(o1[0, 0])
    blocks = sorted({0, 5, 9, 11, nkb - 1} | set(rng.choice(nkb, 8, replace=False).tolist()))
    ref = oa.masked_attention(_np(q[0, 0]), _np(k[0, 0]), _np(v[0, 0]), st, ln, st, ln, keep, blocks=blocks)
    _check_out(o, ref, _rows_of(st, ln, blocks), f"{len(blocks)} query blocks")
    assert (o[st[11]:st[11] + 64] == 0).all()                       # no kept block: zero rows
    assert (o[nv:] == 0).all()
    o2 = bsa.block_sparse_attn_fwd(qd, kd, vd, cd, id_, n_valid=nv)
    assert torch.equal(o1, o2)
    for t in (qd, kd, vd):
        t[:, :, nv:] = float("nan")
    o3 = bsa.block_sparse_attn_fwd(qd, kd, vd, cd, id_, n_valid=nv)
    assert torch.equal(o1, o3)


def _random_partition(rng, n, lens=(0, 1, 7, 17, 33, 64, 65, 100, 150, 230)):
    st, ln, pos = [], [], 0
    while pos < n:
        L = int(min(rng.choice(lens), n - pos))
        st.append(pos)
        ln.append(L)
        pos += L
    return np.array(st, np.int32), np.array(ln, np.int32)


@pytest.mark.parametrize("d,per_head,mode", [(128, False, "any"), (64, True, "any"), (128, True, "any"),
                                             (128, False, "short"), (64, True, "short"), (128, True, "short"),
                                             (128, True, "qshort")])
def test_attn_variable_blocks_random(gpu_lib, d, per_head, mode):
    # "any": query blocks of any length (tiled by 64 rows) and key blocks of
    # any length (runs or gathered 64-row chunks), shared or per head; "short":
    # blocks of at most 64 tokens declared as such (one tile / chunk each);
    # "qshort": short query blocks with gathered key blocks
    bsa = gpu_lib
    H, N, nv = 3, 1100, 1037
    rng = np.random.default_rng(d + per_head + 7 * len(mode))
    say(f"attention variable blocks d={d} per_head={per_head} mode={mode}")
    x = rng.normal(size=(3, 1, H, N, d)).astype(np.float32)
    x[:, :, :, nv:] = 0
    q, k, v = (torch.from_numpy(x[i] * (2.0 if i < 2 else 1.0)).to(torch.bfloat16) for i in range(3))
    heads = range(H) if per_head else [0]
    short_lens = (0, 1, 7, 17, 33, 48, 64, 64, 64)
    parts_q = [_random_partition(rng, nv, short_lens) if mode != "any" else _random_partition(rng, nv)
               for _ in heads]
    parts_k = [_random_partition(rng, nv, short_lens) if mode == "short" else _random_partition(rng, nv)
               for _ in heads]
    mq = 64 if mode != "any" else 0
    mk = 64 if mode == "short" else 0
    nqb = max(len(p[0]) for p in parts_q)
    nkb = max(len(p[0]) for p in parts_k)

    def pad(parts, nb):
        st = np.zeros((len(parts), nb), np.int32)
        ln = np.zeros((len(parts), nb), np.int32)
        for i, (s, l) in enumerate(parts):
            st[i, :len(s)], ln[i, :len(l)] = s, l
            st[i, len(s):] = nv
        return st, ln

    qst, qln = pad(parts_q, nqb)
    kst, kln = pad(parts_k, nkb)
    keep = rng.random((H, nqb, nkb)) < 0.25
    keep[:, :, 0] = True
    if mode == "any":
        # every third query block keeps only key blocks of at most 33 tokens,
        # a chunk each: as runs they take over twice the packed chunks, so
        # these lists are gathered while the others run
        for h in range(H):
            short_k = kln[h if per_head else 0] <= 33
            keep[h, 1::3] = short_k[None] & (rng.random((len(range(1, nqb, 3)), nkb)) < 0.7)
    keep[:, 3, :] = False           # a query block with nothing kept -> zero rows
    cnt = keep.sum(2).astype(np.int32)
    idx = np.full((H, nqb, nkb), -1, np.int32)
    for h in range(H):
        for i in range(nqb):
            ids = np.nonzero(keep[h, i])[0]
            idx[h, i, :len(ids)] = ids
    if per_head:
        qb = bsa.Blocks(torch.from_numpy(qst[None]).cuda(), torch.from_numpy(qln[None]).cuda(), mq)
        kb = bsa.Blocks(torch.from_numpy(kst[None]).cuda(), torch.from_numpy(kln[None]).cuda(), mk)
    else:
        qb = bsa.Blocks(torch.from_numpy(qst[0]).cuda(), torch.from_numpy(qln[0]).cuda(), mq)
        kb = bsa.Blocks(torch.from_numpy(kst[0]).cuda(), torch.from_numpy(kln[0]).cuda(), mk)
    o = bsa.block_sparse_attn_fwd(q.cuda(), k.cuda(), v.cuda(), torch.from_numpy(cnt[None]).cuda(),
                                  torch.from_numpy(idx[None]).cuda(), n_valid=nv, qb=qb, kb=kb)
    o = _np(o)
    if mode == "any":
        # the list of a query block runs as contiguous key runs when they take
        # at most twice the 64-key chunks of packing, else gathered: the case
        # holds both kinds
        kinds = set()
        for h in range(H):
            for i in range(nqb):
                lens = kln[h if per_head else 0][keep[h, i]]
                kinds.add(int(((lens + 63) // 64).sum()) <= 2 * ((int(lens.sum()) + 63) // 64))
        assert kinds == {True, False}
    assert (o[:, :, nv:] == 0).all()
    for h in range(H):
        hi = h if per_head else 0
        ref = oa.masked_attention(_np(q[0, h]), _np(k[0, h]), _np(v[0, h]), qst[hi], qln[hi],
                                  kst[hi], kln[hi], keep[h])
        _check_out(o[0, h], ref, np.arange(nv), f"head {h}")
        s3, l3 = qst[hi][3], qln[hi][3]
        assert (o[0, h, s3:s3 + l3] == 0).all()
