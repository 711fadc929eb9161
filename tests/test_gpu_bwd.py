"""GPU parity of the block-sparse attention backward (and the forward's row
log-normaliser) against the float64 CPU reference in oracle/attention.py.

Tolerance: the kernels round P and dS to bf16 before the second product of
each pair (relative 2^-9 per factor) and store bf16 gradients (another
2^-9), with fp32 accumulation; errors are measured relative to the size of
each gradient: max |g - ref| <= 2e-2 * max(1, max |ref|) and mean
|g - ref| <= 2e-3 * max(1, max |ref|). The row normaliser is fp32 throughout
(one log2 per row): |lse - ref| <= 1e-3 absolute.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from gen import WORKLOADS, generate
from oracle import attention as oa
from oracle import layout as ol
from tests.band import keep_from_lists

pytestmark = pytest.mark.gpu

REL_MAX = 2e-2
REL_MEAN = 2e-3
LSE_ABS = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check_grad(g, ref, rows, what):
    g, ref = g[rows], ref[rows]
    scale = max(1.0, float(np.abs(ref).max()))
    d = np.abs(g - ref)
    say(f"  {what}: max-abs {d.max():.3e} mean-abs {d.mean():.3e} (scale {scale:.3g})")
    assert np.isfinite(g).all(), what
    assert d.max() <= REL_MAX * scale and d.mean() <= REL_MEAN * scale, what


def _lists(keep):
    H, nq, nk = keep.shape
    cnt = keep.sum(2).astype(np.int32)
    idx = np.full((H, nq, nk), -1, np.int32)
    for h in range(H):
        for i in range(nq):
            ids = np.nonzero(keep[h, i])[0]
            idx[h, i, :len(ids)] = ids
    return cnt, idx


def _run_case(bsa, q, k, v, do, cnt, idx, nv, heads=None):
    """GPU forward (with lse) + backward, compared to the oracle per head."""
    H, N = q.shape[1], q.shape[2]
    qd, kd, vd, gd = (t.cuda() for t in (q, k, v, do))
    cd, id_ = torch.from_numpy(cnt[None]).cuda(), torch.from_numpy(idx[None]).cuda()
    o, lse = bsa.block_sparse_attn_fwd_lse(qd, kd, vd, cd, id_, n_valid=nv)
    o_plain = bsa.block_sparse_attn_fwd(qd, kd, vd, cd, id_, n_valid=nv)
    assert torch.equal(o, o_plain)                 # the lse output changes no bit of O
    dq, dk, dv = bsa.block_sparse_attn_bwd(qd, kd, vd, o, gd, lse, cd, id_, n_valid=nv)
    torch.cuda.synchronize()
    dq2, dk2, dv2 = bsa.block_sparse_attn_bwd(qd, kd, vd, o, gd, lse, cd, id_, n_valid=nv)
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)   # deterministic
    st, ln = ol.raster_blocks(nv)
    nb = len(st)
    lse_g, dq, dk, dv = (_np(t)[0] for t in (lse, dq, dk, dv))
    rows = np.arange(nv)
    for h in (range(H) if heads is None else heads):
        keep = keep_from_lists(cnt[h], idx[h], nb)
        args = [_np(t[0, h]) for t in (q, k, v)]
        ref_l = oa.masked_attention_lse(args[0], args[1], st, ln, st, ln, keep)
        fin = np.isfinite(ref_l[rows])
        assert np.array_equal(np.isfinite(lse_g[h][rows]), fin), f"head {h}: -inf rows differ"
        dl = np.abs(lse_g[h][rows][fin] - ref_l[rows][fin])
        say(f"  head {h} lse: max-abs {dl.max() if dl.size else 0:.3e}")
        assert dl.size == 0 or dl.max() <= LSE_ABS
        rq, rk, rv = oa.masked_attention_bwd(*args, _np(do[0, h]), st, ln, st, ln, keep)
        _check_grad(dq[h], rq, rows, f"head {h} dq")
        _check_grad(dk[h], rk, rows, f"head {h} dk")
        _check_grad(dv[h], rv, rows, f"head {h} dv")
    for t in (dq, dk, dv):
        assert (t[:, nv:] == 0).all()
    assert np.isneginf(lse_g[:, nv:]).all()


@pytest.mark.parametrize("H,N,nv,d", [(2, 256, 256, 64), (2, 704, 650, 128), (1, 1088, 1030, 64)])
def test_bwd_random_masks(gpu_lib, H, N, nv, d):
    say(f"backward random masks H={H} N={N} n_valid={nv} d={d}")
    rng = np.random.default_rng(N + d)
    x = rng.normal(size=(4, 1, H, N, d)).astype(np.float32)
    x[:, :, :, nv:] = 0
    q, k, v, do = (torch.from_numpy(x[i] * (2.0 if i < 2 else 1.0)).to(torch.bfloat16) for i in range(4))
    nb = -(-nv // 64)
    keep = rng.random((H, nb, nb)) < 0.35
    keep[:, :, 0] |= ~keep.any(2)
    keep[:, 0, :] = True                            # a dense row
    if nb > 3:
        keep[:, 2, :] = False                       # a row that keeps nothing
        keep[:, :, nb - 2] = False                  # a key block nobody keeps
    cnt, idx = _lists(keep)
    _run_case(gpu_lib, q, k, v, do, cnt, idx, nv)


def test_bwd_mask_stage_lists(gpu_lib):
    # the lists the mask stage builds on the Fourier-feature inputs (the
    # tiny workload and the first 4096 tokens of the 480p layer, two heads)
    bsa = gpu_lib
    for key, N in (("tiny", None), ("wan480", 4096)):
        w = WORKLOADS[key]
        q, k, v = generate(w, heads=[0, 1])
        if N is not None:
            q, k, v = (t[:, :, :N].contiguous() for t in (q, k, v))
        N = q.shape[2]
        nv = min(w.n_valid, N)
        say(f"backward on mask-stage lists: {key} N={N}")
        do = torch.randn(q.shape, generator=torch.Generator().manual_seed(7)).to(torch.bfloat16)
        cnt, idx = bsa.build_block_mask(q.cuda(), k.cuda(), w.thr, n_valid=nv)
        _run_case(bsa, q, k, v, do, cnt.cpu().numpy()[0], idx.cpu().numpy()[0], nv)


def test_bwd_wan480_full_layer_sampled(gpu_lib):
    # the whole 480p layer (12 heads, 32,760 tokens, the mask stage's lists) in
    # the launch the bench times; sampled query blocks' dQ and sampled key
    # blocks' dK, dV against the oracle (each from every query block that
    # kept that key block), on two heads
    bsa = gpu_lib
    w = WORKLOADS["wan480"]
    q, k, v = generate(w)
    nv = w.n_valid
    say("backward, full 480p layer, sampled blocks")
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    do[:, :, nv:] = 0
    qd, kd, vd, gd = (t.cuda() for t in (q, k, v, do))
    cnt, idx = bsa.build_block_mask(qd, kd, w.thr, n_valid=nv)
    o, lse = bsa.block_sparse_attn_fwd_lse(qd, kd, vd, cnt, idx, n_valid=nv)
    dq, dk, dv = bsa.block_sparse_attn_bwd(qd, kd, vd, o, gd, lse, cnt, idx, n_valid=nv)
    torch.cuda.synchronize()
    cnt, idx = cnt.cpu().numpy()[0], idx.cpu().numpy()[0]
    dq, dk, dv = (_np(t)[0] for t in (dq, dk, dv))
    for t in (dq, dk, dv):
        assert (t[:, nv:] == 0).all()
    st, ln = ol.raster_blocks(nv)
    nb = len(st)
    rng = np.random.default_rng(9)
    for h in (2, 9):
        keep = keep_from_lists(cnt[h], idx[h], nb)
        args = [_np(t[0, h]) for t in (q, k, v, do)]
        qi = sorted(set(rng.choice(nb, 3, replace=False).tolist()) | {nb - 1})
        rq, _, _ = oa.masked_attention_bwd(*args, st[qi], ln[qi], st, ln, keep[qi])
        rows = np.concatenate([np.arange(st[i], st[i] + ln[i]) for i in qi])
        _check_grad(dq[h], rq, rows, f"head {h} dq (query blocks {qi})")
        # key blocks: a well-kept one and the last (ragged) one
        for J in (int(np.argmax(keep.sum(0))), nb - 1):
            users = np.nonzero(keep[:, J])[0]
            if len(users) == 0:
                continue
            _, rk, rv = oa.masked_attention_bwd(*args, st[users], ln[users], st, ln, keep[users])
            krows = np.arange(st[J], st[J] + ln[J])
            _check_grad(dk[h], rk, krows, f"head {h} dk (key block {J}, {len(users)} query blocks)")
            _check_grad(dv[h], rv, krows, f"head {h} dv (key block {J})")


def test_bwd_hunyuan720_sampled(gpu_lib):
    # the 720p layer (24 heads, 118,800 tokens, 1857 key blocks): the
    # transposed lists over 59 bit-words per row, sampled blocks of one head
    bsa = gpu_lib
    w = WORKLOADS["hunyuan720"]
    q, k, v = generate(w)
    nv = w.n_valid
    say("backward, 720p layer, sampled blocks of head 13")
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(6)).to(torch.bfloat16)
    do[:, :, nv:] = 0
    qd, kd, vd, gd = (t.cuda() for t in (q, k, v, do))
    cnt, idx = bsa.build_block_mask(qd, kd, w.thr, n_valid=nv)
    o, lse = bsa.block_sparse_attn_fwd_lse(qd, kd, vd, cnt, idx, n_valid=nv)
    dq, dk, dv = bsa.block_sparse_attn_bwd(qd, kd, vd, o, gd, lse, cnt, idx, n_valid=nv)
    torch.cuda.synchronize()
    h = 13
    cnt, idx = cnt[0, h].cpu().numpy(), idx[0, h].cpu().numpy()
    dq, dk, dv = (_np(t[0, h]) for t in (dq, dk, dv))
    assert (dq[nv:] == 0).all() and (dk[nv:] == 0).all() and (dv[nv:] == 0).all()
    st, ln = ol.raster_blocks(nv)
    nb = len(st)
    keep = keep_from_lists(cnt, idx, nb)
    args = [_np(t[0, h]) for t in (q, k, v, do)]
    qi = [int(np.argmax(cnt)), nb - 1]
    rq, _, _ = oa.masked_attention_bwd(*args, st[qi], ln[qi], st, ln, keep[qi])
    rows = np.concatenate([np.arange(st[i], st[i] + ln[i]) for i in qi])
    _check_grad(dq, rq, rows, f"dq (query blocks {qi}, {cnt[qi].tolist()} kept)")
    J = nb - 1
    users = np.nonzero(keep[:, J])[0]
    if len(users):
        _, rk, rv = oa.masked_attention_bwd(*args, st[users], ln[users], st, ln, keep[users])
        krows = np.arange(st[J], st[J] + ln[J])
        _check_grad(dk, rk, krows, f"dk (key block {J}, {len(users)} query blocks)")
        _check_grad(dv, rv, krows, f"dv (key block {J})")


def _short_partition(rng, n, lens=(0, 1, 7, 17, 33, 48, 64, 64, 64)):
    st, ln, pos = [], [], 0
    while pos < n:
        L = int(min(rng.choice(lens), n - pos))
        st.append(pos)
        ln.append(L)
        pos += L
    return np.array(st, np.int32), np.array(ln, np.int32)


@pytest.mark.parametrize("H,N,nv,d", [(2, 704, 650, 128), (2, 320, 300, 64)])
def test_bwd_bounded_blocks_random(gpu_lib, H, N, nv, d):
    # query and key blocks of at most 64 tokens (empty, ragged and full ones)
    # that partition the valid tokens, per head
    bsa = gpu_lib
    say(f"backward over bounded blocks H={H} N={N} n_valid={nv} d={d}")
    rng = np.random.default_rng(N * 3 + d)
    x = rng.normal(size=(4, 1, H, N, d)).astype(np.float32)
    x[:, :, :, nv:] = 0
    q, k, v, do = (torch.from_numpy(x[i] * (2.0 if i < 2 else 1.0)).to(torch.bfloat16) for i in range(4))
    parts_q = [_short_partition(rng, nv) for _ in range(H)]
    parts_k = [_short_partition(rng, nv) for _ in range(H)]
    nqb, nkb = max(len(p[0]) for p in parts_q), max(len(p[0]) for p in parts_k)

    def pad(parts, nb):
        st = np.full((H, nb), nv, np.int32)
        ln = np.zeros((H, nb), np.int32)
        for h, (s_, l_) in enumerate(parts):
            st[h, :len(s_)], ln[h, :len(l_)] = s_, l_
        return st, ln

    qst, qln = pad(parts_q, nqb)
    kst, kln = pad(parts_k, nkb)
    keep = rng.random((H, nqb, nkb)) < 0.3
    keep[:, :, 0] |= ~keep.any(2)
    cnt = keep.sum(2).astype(np.int32)
    idx = np.full((H, nqb, nkb), -1, np.int32)
    for h in range(H):
        for i in range(nqb):
            ids = np.nonzero(keep[h, i])[0]
            idx[h, i, :len(ids)] = ids
    qb = bsa.Blocks(torch.from_numpy(qst[None]).cuda(), torch.from_numpy(qln[None]).cuda(), 64)
    kb = bsa.Blocks(torch.from_numpy(kst[None]).cuda(), torch.from_numpy(kln[None]).cuda(), 64)
    qd, kd, vd, gd = (t.cuda() for t in (q, k, v, do))
    cd, id_ = torch.from_numpy(cnt[None]).cuda(), torch.from_numpy(idx[None]).cuda()
    o, lse = bsa.block_sparse_attn_fwd_lse(qd, kd, vd, cd, id_, n_valid=nv, qb=qb, kb=kb)
    dq, dk, dv = bsa.block_sparse_attn_bwd(qd, kd, vd, o, gd, lse, cd, id_, n_valid=nv, qb=qb, kb=kb)
    dq2, dk2, dv2 = bsa.block_sparse_attn_bwd(qd, kd, vd, o, gd, lse, cd, id_, n_valid=nv, qb=qb, kb=kb)
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    lse_g, dq, dk, dv = (_np(t)[0] for t in (lse, dq, dk, dv))
    rows = np.arange(nv)
    for h in range(H):
        args = [_np(t[0, h]) for t in (q, k, v, do)]
        ref_l = oa.masked_attention_lse(args[0], args[1], qst[h], qln[h], kst[h], kln[h], keep[h])
        fin = np.isfinite(ref_l[rows])
        assert np.array_equal(np.isfinite(lse_g[h][rows]), fin)
        assert np.abs(lse_g[h][rows][fin] - ref_l[rows][fin]).max() <= LSE_ABS
        rq, rk, rv = oa.masked_attention_bwd(*args, qst[h], qln[h], kst[h], kln[h], keep[h])
        _check_grad(dq[h], rq, rows, f"head {h} dq")
        _check_grad(dk[h], rk, rows, f"head {h} dk")
        _check_grad(dv[h], rv, rows, f"head {h} dv")
    for t in (dq, dk, dv):
        assert (t[:, nv:] == 0).all()


def test_bwd_fractal_patches_wan480_sampled(gpu_lib):
    # the hybrid layout: fractal patches (588 blocks of 24..64 tokens), the CDF
    # mask OR the sliding-tile window, on the permuted 480p layer
    import block_sparse_attention_avg_amd.pipelines as pl
    bsa = gpu_lib
    w = WORKLOADS["wan480_fractal_sta"]
    q, k, v = generate(w, heads=[0, 5])
    nv = w.n_valid
    say("backward over fractal patches, 480p layer, sampled blocks")
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(8)).to(torch.bfloat16)
    do[:, :, nv:] = 0
    lay = pl.fractal_layout(w.T, w.Hl, w.Wl, w.patch, w.N, "cuda")
    qp, kp, vp, gp = (bsa.permute_tokens(t.cuda(), lay.perm) for t in (q, k, v, do))
    cnt, idx = bsa.build_block_mask(qp, kp, w.thr, window=(*lay.grid, *w.window), n_valid=nv,
                                    qb=lay.blocks, kb=lay.blocks)
    o, lse = bsa.block_sparse_attn_fwd_lse(qp, kp, vp, cnt, idx, n_valid=nv, qb=lay.blocks, kb=lay.blocks)
    dq, dk, dv = bsa.block_sparse_attn_bwd(qp, kp, vp, o, gp, lse, cnt, idx, n_valid=nv, qb=lay.blocks,
                                           kb=lay.blocks)
    torch.cuda.synchronize()
    perm, st, ln, _ = ol.fractal_order(w.T, w.Hl, w.Wl, w.patch, w.N)
    nb = len(st)
    cnt, idx = cnt.cpu().numpy()[0], idx.cpu().numpy()[0]
    dq, dk, dv = (_np(t)[0] for t in (dq, dk, dv))
    rng = np.random.default_rng(12)
    for h in range(2):
        keep = keep_from_lists(cnt[h], idx[h], nb)
        args = [_np(t[0, h])[perm] for t in (q, k, v, do)]
        qi = sorted(set(rng.choice(nb, 3, replace=False).tolist()) | {nb - 1})
        rq, _, _ = oa.masked_attention_bwd(*args, st[qi], ln[qi], st, ln, keep[qi])
        rows = np.concatenate([np.arange(st[i], st[i] + ln[i]) for i in qi])
        _check_grad(dq[h], rq, rows, f"head {h} dq (patches {qi})")
        J = int(np.argmin(ln))                       # a short edge patch
        users = np.nonzero(keep[:, J])[0]
        _, rk, rv = oa.masked_attention_bwd(*args, st[users], ln[users], st, ln, keep[users])
        krows = np.arange(st[J], st[J] + ln[J])
        _check_grad(dk[h], rk, krows, f"head {h} dk (patch {J} of {ln[J]} tokens, {len(users)} query patches)")
        _check_grad(dv[h], rv, krows, f"head {h} dv (patch {J})")


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_max_key_blocks(gpu_lib, d):
    # the supported maximum of 8192 query and key blocks: neither
    # longest-first order (query tiles by kept count, key tiles by user
    # count) fits its 64 KiB of LDS, so both tile kinds run in block order;
    # the transposed lists span 256 bit-words per key block. Random 1 %
    # lists with a dense row, a row keeping nothing, a key block kept by
    # every 16th query block and the ragged last block; dQ of sampled query
    # blocks and dK, dV of sampled key blocks (every query block that keeps
    # them, whole) against the reference, then a repeat run
    bsa = gpu_lib
    nkb = 8192
    N = nkb * 64
    nv = N - 37
    rng = np.random.default_rng(9000 + d)
    say(f"backward, max key blocks d={d} N={N} n_valid={nv}")
    x = [rng.normal(size=(N, d)).astype(np.float32) for _ in range(4)]
    for t in x:
        t[nv:] = 0
    q, k, v, do = (torch.from_numpy(t[None, None] * (1.5 if i < 2 else 1.0)).to(torch.bfloat16)
                   for i, t in enumerate(x))
    del x
    st, ln = ol.raster_blocks(nv)
    assert len(st) == nkb
    keep = rng.random((nkb, nkb), dtype=np.float32) < 0.01
    keep[:, 0] |= ~keep.any(1)
    keep[5, :] = True                                  # a dense row
    keep[11, :] = False                                # a row keeping nothing
    keep[::16, 777] = True                             # a key block 512 query blocks keep
    keep[11, 777] = False
    cnt, idx = _lists(keep[None])
    qd, kd, vd, gd = (t.cuda() for t in (q, k, v, do))
    cd, id_ = torch.from_numpy(cnt[None]).cuda(), torch.from_numpy(idx[None]).cuda()
    del idx
    o, lse = bsa.block_sparse_attn_fwd_lse(qd, kd, vd, cd, id_, n_valid=nv)
    g1 = bsa.block_sparse_attn_bwd(qd, kd, vd, o, gd, lse, cd, id_, n_valid=nv)
    torch.cuda.synchronize()
    g2 = bsa.block_sparse_attn_bwd(qd, kd, vd, o, gd, lse, cd, id_, n_valid=nv)
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))            # deterministic
    dq, dk, dv = (_np(t[0, 0]) for t in g1)
    del g1, g2
    assert (dq[nv:] == 0).all() and (dk[nv:] == 0).all() and (dv[nv:] == 0).all()
    assert (dq[st[11]:st[11] + 64] == 0).all()
    args = [_np(t[0, 0]) for t in (q, k, v, do)]
    qi = sorted({5, 11, nkb - 1} | set(rng.choice(nkb, 4, replace=False).tolist()))
    rq, _, _ = oa.masked_attention_bwd(*args, st[qi], ln[qi], st, ln, keep[qi])
    rows = np.concatenate([np.arange(st[i], st[i] + ln[i]) for i in qi])
    _check_grad(dq, rq, rows, f"dq (query blocks {qi})")
    for J in (777, nkb - 1, int(rng.integers(1, nkb - 1))):
        users = np.nonzero(keep[:, J])[0]
        _, rk, rv = oa.masked_attention_bwd(*args, st[users], ln[users], st, ln, keep[users])
        krows = np.arange(st[J], st[J] + ln[J])
        _check_grad(dk, rk, krows, f"dk (key block {J}, {len(users)} query blocks)")
        _check_grad(dv, rv, krows, f"dv (key block {J})")
