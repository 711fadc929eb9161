"""The C ABI library loads without a GPU, exports every declared entry point,
and rejects invalid arguments on the host before any launch (no GPU)."""

import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_attention_avg_amd as bsa
from oracle import layout as ol

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return bsa.load()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(bsa.EXPORTS) == names


def test_version_and_strerror(lib):
    assert lib.bsa_abi_version() == 2
    for code in range(5):
        assert lib.bsa_strerror(code).decode()
    assert lib.bsa_strerror(99).decode() == "unknown status"


def _err(lib):
    return lib.bsa_last_error_message().decode()


def test_argument_validation_before_launch(lib):
    P = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    # unsupported head dim
    assert lib.bsa_pool_blocks(P, 1, 1, 64, 96, 64, 64, None, P, None) == 2
    assert "head dim" in _err(lib)
    # n_valid > N
    assert lib.bsa_pool_blocks(P, 1, 1, 64, 64, 65, 64, None, P, None) == 1
    # uniform blocks must be 64 tokens
    assert lib.bsa_pool_blocks(P, 1, 1, 64, 64, 64, 32, None, P, None) == 2
    # null pointer
    assert lib.bsa_pool_blocks(None, 1, 1, 64, 64, 64, 64, None, P, None) == 1
    # misaligned
    assert lib.bsa_pool_blocks(ctypes.c_void_p(18), 1, 1, 64, 64, 64, 64, None, P, None) == 1
    # thr outside [0, 1] and NaN
    for thr in (-0.1, 1.5, float("nan")):
        assert lib.bsa_select_blocks(P, P, 1, 1, 4, 4, 64, None, None, thr, 0.0, None, P, P, 4, None) == 1
    # kv_stride too small
    assert lib.bsa_select_blocks(P, P, 1, 1, 4, 4, 64, None, None, 0.1, 0.0, None, P, P, 3, None) == 3
    # too many key blocks
    assert lib.bsa_select_blocks(P, P, 1, 1, 4, 9000, 64, None, None, 0.1, 0.0, None, P, P, 9000, None) == 2
    # window grid mismatch
    w = bsa._Window(2, 2, 2, 1, 1, 1)
    assert lib.bsa_select_blocks(P, P, 1, 1, 4, 4, 64, None, None, 0.1, 0.0, ctypes.byref(w), P, P, 4, None) == 1
    assert "window" in _err(lib)
    # workspace too small
    assert lib.bsa_build_block_mask(P, P, 1, 1, 128, 64, 128, 64, None, None, 0.1, None, P, P, 2, P, 16, None) == 3
    # attention: variable query blocks need a workspace
    blk = bsa._Blocks(2, 0, 16, 16)
    assert lib.bsa_block_sparse_attn_fwd(P, P, P, P, 1, 1, 128, 64, 128, 64, ctypes.byref(blk), None,
                                         P, P, 2, 0.0, None, 0, None) == 3
    # k-means: C out of range / larger than n_valid / no workspace
    assert lib.bsa_kmeans(P, 1, 1, 128, 64, 128, 2000, 10, P, P, P, P, P, 1 << 30, None) == 2
    assert lib.bsa_kmeans(P, 1, 1, 128, 64, 100, 101, 10, P, P, P, P, P, 1 << 30, None) == 1
    assert lib.bsa_kmeans(P, 1, 1, 128, 64, 128, 8, 10, P, P, P, P, None, 0, None) == 3
    # permute: in place is rejected
    assert lib.bsa_permute_tokens(P, P, P, 1, 1, 8, 64, 0, None) == 1


def test_argument_validation_newer_entry_points(lib):
    P = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    # forward with row normaliser: lse is required; variable blocks are not supported there
    assert lib.bsa_block_sparse_attn_fwd_lse(P, P, P, P, None, 1, 1, 128, 64, 128, 64, None, None, P, P, 2,
                                             0.0, P, 1 << 20, None) == 1
    # backward: uniform 64-token blocks only, pointers, workspace
    assert lib.bsa_block_sparse_attn_bwd(P, P, P, P, P, P, 1, 1, 128, 64, 128, 32, None, None, P, P, 2, 0.0, P, P,
                                         P, P, 1 << 30, None) == 2
    assert lib.bsa_block_sparse_attn_bwd(P, P, P, P, None, P, 1, 1, 128, 64, 128, 64, None, None, P, P, 2, 0.0, P,
                                         P, P, P, 1 << 30, None) == 1
    assert lib.bsa_block_sparse_attn_bwd(P, P, P, P, P, P, 1, 1, 128, 64, 128, 64, None, None, P, P, 2, 0.0, P, P,
                                         P, P, 16, None) == 3
    assert "workspace" in _err(lib)
    # block descriptors without a length bound are refused
    blk = bsa._Blocks(2, 0, 16, 16, 0)
    assert lib.bsa_block_sparse_attn_bwd(P, P, P, P, P, P, 1, 1, 128, 64, 128, 64, ctypes.byref(blk),
                                         ctypes.byref(blk), P, P, 2, 0.0, P, P, P, P, 1 << 30, None) == 2
    assert "max_len" in _err(lib)
    # warm-started k-means: rounds, tolerance, the move counts are required
    assert lib.bsa_kmeans_warm(P, 1, 1, 128, 64, 128, 8, 0, 0, P, P, P, P, P, 1 << 30, None) == 1
    assert lib.bsa_kmeans_warm(P, 1, 1, 128, 64, 128, 8, 5, -1, P, P, P, P, P, 1 << 30, None) == 1
    assert lib.bsa_kmeans_warm(P, 1, 1, 128, 64, 128, 8, 5, 0, P, P, P, None, P, 1 << 30, None) == 1
    assert lib.bsa_kmeans_warm(P, 1, 1, 128, 64, 128, 8, 5, 0, P, P, P, P, None, 0, None) == 3
    # tile statistics and recall
    assert lib.bsa_attention_tile_stats(P, P, P, 1, 1, 128, 96, 128, 0.0, P, P, P, None) == 2
    assert lib.bsa_attention_tile_stats(P, P, None, 1, 1, 128, 64, 128, 0.0, P, P, P, None) == 1
    assert lib.bsa_mask_recall(P, P, P, P, 9000, 1, 1, 4, 9000, P, P, None) == 2
    assert lib.bsa_mask_recall(P, P, P, P, 0, 1, 1, 4, 4, P, P, None) == 1
    assert lib.bsa_mask_recall(P, None, P, P, 4, 1, 1, 4, 4, P, P, None) == 1
    # list validator
    assert lib.bsa_check_mask(P, P, 1, 1, 4, 0, 4, P, None) == 1
    assert lib.bsa_check_mask(P, P, 1, 1, 4, 4, 0, P, None) == 1
    assert lib.bsa_check_mask(P, None, 1, 1, 4, 4, 4, P, None) == 1
    assert lib.bsa_check_mask(P, P, 1, 1, 4, 4, 4, None, None) == 1


def test_workspace_queries(lib):
    assert lib.bsa_build_block_mask_workspace(1, 12, 512, 512, 128) == 2 * 12 * 512 * 128 * 4
    assert lib.bsa_block_sparse_attn_fwd_workspace(1, 12, 512, None) >= 12 * 513 * 4
    blk = bsa._Blocks(588, 0, 16, 16)
    assert lib.bsa_block_sparse_attn_fwd_workspace(1, 12, 588, ctypes.byref(blk)) >= 12 * 589 * 4
    assert lib.bsa_kmeans_workspace(1, 12, 32768, 256, 128) > 0
    assert lib.bsa_cluster_order_workspace(1, 12, 32768, 256) > 0


@pytest.mark.parametrize("T,Hl,Wl,P,N", [(21, 30, 52, 8, 32768), (3, 5, 7, 2, 110), (2, 8, 8, 8, 128)])
def test_fractal_order_host_function_matches_reference(T, Hl, Wl, P, N):
    perm, st, ln, co = bsa.fractal_order(T, Hl, Wl, P, N)
    rp, rs, rl, rc = ol.fractal_order(T, Hl, Wl, P, N)
    assert np.array_equal(perm.numpy(), rp) and np.array_equal(st.numpy(), rs)
    assert np.array_equal(ln.numpy(), rl) and np.array_equal(co.numpy(), rc)


@pytest.mark.parametrize("T,Hl,Wl,f,N", [(21, 30, 52, (2, 4, 8), 32768), (21, 30, 52, (4, 4, 4), 32768),
                                         (5, 6, 9, (3, 2, 5), 280), (2, 3, 3, (4, 4, 4), 18)])
def test_tile_order_host_function_matches_reference(T, Hl, Wl, f, N):
    perm, st, ln, co = bsa.tile_order(T, Hl, Wl, *f, N)
    rp, rs, rl, rc = ol.tile_order(T, Hl, Wl, *f, N)
    assert np.array_equal(perm.numpy(), rp) and np.array_equal(st.numpy(), rs)
    assert np.array_equal(ln.numpy(), rl) and np.array_equal(co.numpy(), rc)


def test_tile_order_errors(lib):
    perm = (ctypes.c_int32 * 256)()
    st = (ctypes.c_int32 * 4)()
    ln = (ctypes.c_int32 * 4)()
    nb = ctypes.c_int(0)
    args = [ctypes.cast(perm, ctypes.c_void_p), ctypes.cast(st, ctypes.c_void_p), ctypes.cast(ln, ctypes.c_void_p),
            None, 4, ctypes.byref(nb)]
    assert lib.bsa_tile_order(4, 8, 8, 2, 4, 4, 256, *args) == 3 and nb.value == 8       # ENOSPC
    assert lib.bsa_tile_order(4, 8, 8, 0, 4, 4, 256, *args) == 1                         # EINVAL
    assert lib.bsa_tile_order(4, 8, 8, 2, 4, 4, 255, *args) == 1                         # N too small
    assert lib.bsa_tile_order(1, 8, 8, 1, 4, 4, 64, *args) == 0 and nb.value == 4


def test_fractal_order_capacity(lib):
    perm = (ctypes.c_int32 * 256)()
    st = (ctypes.c_int32 * 4)()
    ln = (ctypes.c_int32 * 4)()
    nb = ctypes.c_int(0)
    rc = lib.bsa_fractal_order(4, 8, 8, 4, 256, ctypes.cast(perm, ctypes.c_void_p), ctypes.cast(st, ctypes.c_void_p),
                               ctypes.cast(ln, ctypes.c_void_p), None, 4, ctypes.byref(nb))
    assert rc == 3 and nb.value == 16


def test_noalloc_capacity_is_checked_before_any_launch(lib):
    # past the fixed scratch the allocation-free forward refuses with
    # BSA_ENOSPC before touching the GPU (dummy host pointers are never used)
    cap = lib.bsa_block_sparse_attn_fwd_noalloc_capacity() // 4
    assert cap == 1 << 18
    buf = (ctypes.c_uint8 * 64)()
    p = (ctypes.addressof(buf) + 15) // 16 * 16
    H, nb = 64, cap // 64 + 1
    st = lib.bsa_block_sparse_attn_fwd_noalloc(p, p, p, p, 1, H, nb * 64, 128, nb * 64, 64, None, None, p, p, nb,
                                               ctypes.c_float(0.0), None)
    assert st == 3
    assert b"scratch" in lib.bsa_last_error_message()
    # bad shapes are still refused first
    assert lib.bsa_block_sparse_attn_fwd_noalloc(p, p, p, p, 0, H, 64, 128, 64, 64, None, None, p, p, 1,
                                                 ctypes.c_float(0.0), None) == 1
