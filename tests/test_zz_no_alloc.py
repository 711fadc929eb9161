"""The allocation-free attention forward against the forward with a workspace.

bsa_block_sparse_attn_fwd_noalloc runs the same kernels as
bsa_block_sparse_attn_fwd with the workspace table in a fixed device array of
the library, so its output must equal that entry point's bit for bit. Two
calls in a row, the second on a smaller problem (the array keeps the first
call's contents), both through the C ABI; then a problem past the array's
capacity is refused before any launch.
"""

import ctypes

import numpy as np
import pytest
import torch

from oracle import attention as oa, layout as ol

pytestmark = pytest.mark.gpu


def _case(rng, H, N, nv, d, density):
    x = rng.normal(size=(3, 1, H, N, d)).astype(np.float32)
    x[:, :, :, nv:] = 0
    q, k, v = (torch.from_numpy(t).to(torch.bfloat16) for t in x)
    nb = -(-nv // 64)
    cnt = np.zeros((1, H, nb), np.int32)
    idx = np.zeros((1, H, nb, nb), np.int32)
    for h in range(H):
        for r in range(nb):
            ids = np.nonzero(rng.random(nb) < density)[0]
            cnt[0, h, r] = len(ids)
            idx[0, h, r, :len(ids)] = ids
    return q, k, v, cnt, idx, nb


def _noalloc(bsa, q, k, v, cnt, idx, nv):
    lib = bsa.load()
    B, H, N, d = q.shape
    o = torch.full_like(q, float("nan"))
    st = lib.bsa_block_sparse_attn_fwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, N, d, nv, 64, None, None,
        cnt.data_ptr(), idx.data_ptr(), idx.shape[-1], ctypes.c_float(0.0),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.bsa_last_error_message().decode()
    return o


def test_noalloc_matches_workspace_entry_point(gpu_lib):
    bsa = gpu_lib
    rng = np.random.default_rng(77)
    for (H, N, nv, d, dens) in [(6, 64 * 300, 64 * 300 - 37, 128, 0.2), (2, 64 * 40, 64 * 40 - 5, 64, 0.5)]:
        q, k, v, cnt, idx, nb = _case(rng, H, N, nv, d, dens)
        print(f"noalloc H={H} N={N} n_valid={nv} d={d}", flush=True)
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        cd, id_ = torch.from_numpy(cnt).cuda(), torch.from_numpy(idx).cuda()
        ref = bsa.block_sparse_attn_fwd(qd, kd, vd, cd, id_, n_valid=nv)
        got = _noalloc(bsa, qd, kd, vd, cd, id_, nv)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        # and against the CPU reference on a few query blocks of head 0
        st, ln = ol.raster_blocks(nv)
        keep = np.zeros((nb, nb), bool)
        for r in range(nb):
            keep[r, idx[0, 0, r, :cnt[0, 0, r]]] = True
        blocks = [0, nb // 2, nb - 1]
        want = oa.masked_attention(*(t[0, 0].double().numpy() for t in (q, k, v)), st, ln, st, ln, keep,
                                   blocks=blocks)
        g = got[0, 0].float().cpu().numpy()
        for b in blocks:
            rows = slice(st[b], st[b] + ln[b])
            assert np.abs(g[rows] - want[rows]).max() <= 2e-2
        assert (g[nv:] == 0).all()


def test_noalloc_refuses_problems_past_its_capacity(gpu_lib):
    lib = gpu_lib.load()
    cap = lib.bsa_block_sparse_attn_fwd_noalloc_capacity() // 4
    H, nb = 64, cap // 64 + 1             # H * (nb + 1) > cap
    dummy = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    p = dummy.data_ptr()
    st = lib.bsa_block_sparse_attn_fwd_noalloc(p, p, p, p, 1, H, nb * 64, 128, nb * 64, 64, None, None, p, p, nb,
                                               ctypes.c_float(0.0), None)
    assert st == 3                        # BSA_ENOSPC, nothing launched
    assert "scratch" in lib.bsa_last_error_message().decode()
