"""Python binding of libbsa, the gfx950 block-sparse attention library.

Thin ctypes wrappers with the names of the C entry points (without the
``bsa_`` prefix). They only check tensor dtypes/devices/shapes, allocate
outputs and workspaces with torch, and pass raw device pointers plus the
current HIP stream; every step of the computation runs in the library's HIP
kernels. There is no fallback: if ``libbsa.so`` is missing, ``load()`` raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsa.so")
_lib = None

BSA_OK = 0


class BsaError(RuntimeError):
    pass


class _Blocks(ctypes.Structure):
    _fields_ = [("nblocks", ctypes.c_int32), ("per_head", ctypes.c_int32),
                ("start", ctypes.c_void_p), ("len", ctypes.c_void_p), ("max_len", ctypes.c_int32)]


class _Window(ctypes.Structure):
    _fields_ = [("nt", ctypes.c_int32), ("ny", ctypes.c_int32), ("nx", ctypes.c_int32),
                ("rt", ctypes.c_int32), ("ry", ctypes.c_int32), ("rx", ctypes.c_int32)]


_I, _F, _P, _Z = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

_SIGS = {
    "bsa_abi_version": ([], _I),
    "bsa_lds_swizzle": ([_I, _I], _I),
    "bsa_strerror": ([_I], ctypes.c_char_p),
    "bsa_last_error_message": ([], ctypes.c_char_p),
    "bsa_pool_blocks": ([_P, _I, _I, _I, _I, _I, _I, _P, _P, _P], _I),
    "bsa_select_blocks": ([_P, _P, _I, _I, _I, _I, _I, _P, _P, _F, _F, _P, _P, _P, _I, _P], _I),
    "bsa_build_block_mask_workspace": ([_I, _I, _I, _I, _I], _Z),
    "bsa_build_block_mask": ([_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _F, _P, _P, _P, _I, _P, _Z, _P], _I),
    "bsa_build_centroid_mask": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _P, _P, _I, _P], _I),
    "bsa_block_sparse_attn_fwd_workspace": ([_I, _I, _I, _P], _Z),
    "bsa_block_sparse_attn_fwd": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _F, _P, _Z, _P], _I),
    "bsa_block_sparse_attn_fwd_noalloc_capacity": ([], _Z),
    "bsa_block_sparse_attn_fwd_noalloc": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _F, _P], _I),
    "bsa_block_sparse_attn_fwd_lse": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _F, _P, _Z,
                                       _P], _I),
    "bsa_block_sparse_attn_bwd_workspace": ([_I, _I, _I, ctypes.POINTER(_Blocks), ctypes.POINTER(_Blocks)], _Z),
    "bsa_block_sparse_attn_bwd": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.POINTER(_Blocks),
                                   ctypes.POINTER(_Blocks), _P, _P, _I, _F, _P, _P, _P, _P,
                                   _Z, _P], _I),
    "bsa_permute_tokens": ([_P, _P, _P, _I, _I, _I, _I, _I, _P], _I),
    "bsa_unpermute_tokens": ([_P, _P, _P, _I, _I, _I, _I, _I, _P], _I),
    "bsa_fractal_order": ([_I, _I, _I, _I, _I, _P, _P, _P, _P, _I, ctypes.POINTER(_I)], _I),
    "bsa_tile_order": ([_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, ctypes.POINTER(_I)], _I),
    "bsa_kmeans_workspace": ([_I, _I, _I, _I, _I], _Z),
    "bsa_kmeans": ([_P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _Z, _P], _I),
    "bsa_attention_tile_stats": ([_P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P], _I),
    "bsa_mask_recall": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P], _I),
    "bsa_check_mask": ([_P, _P, _I, _I, _I, _I, _I, _P, _P], _I),
    "bsa_kmeans_warm": ([_P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _Z, _P], _I),
    "bsa_cluster_order_workspace": ([_I, _I, _I, _I], _Z),
    "bsa_cluster_order": ([_P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _Z, _P], _I),
}

EXPORTS = tuple(_SIGS)


def load(path: Optional[str] = None):
    """Loads libbsa.so (once). Raises if it is missing: there is no fallback.

    The path defaults to the in-tree build; BSA_LIBRARY names another build of
    the same library (the host-sanitized one that the CPU tests run under).
    """
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("BSA_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise BsaError(f"{path} not found; build it with `python -m block_sparse_attention_avg_amd._build`")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != BSA_OK:
        lib = load()
        msg = lib.bsa_last_error_message().decode()
        raise BsaError(f"{what}: {lib.bsa_strerror(status).decode()} ({status}): {msg}")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev_tensor(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _qkv(t: torch.Tensor, name: str):
    _dev_tensor(t, torch.bfloat16, name)
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, N, d]")
    return t.shape


class Blocks:
    """Block descriptors: int32 device tensors ``start`` and ``length`` of shape
    [nblocks] (shared by all heads) or [B, H, nblocks] (per head). ``max_len``
    (1..64) is a bound on every length the caller vouches for; it lets the
    attention take each block as one tile (0: any length)."""

    def __init__(self, start: torch.Tensor, length: torch.Tensor, max_len: int = 0):
        if start.shape != length.shape:
            raise ValueError("start and length must have the same shape")
        _dev_tensor(start, torch.int32, "start")
        _dev_tensor(length, torch.int32, "length")
        self.start, self.length = start, length
        self.per_head = start.dim() > 1
        self.nblocks = start.shape[-1]
        self.max_len = int(max_len)

    def _c(self):
        return _Blocks(self.nblocks, 1 if self.per_head else 0, self.start.data_ptr(), self.length.data_ptr(),
                       self.max_len)


def _blocks_ref(b: Optional[Blocks]):
    return None if b is None else ctypes.byref(b._c())


def _nblocks(b: Optional[Blocks], n_valid: int, block: int) -> int:
    return b.nblocks if b is not None else -(-n_valid // block)


def _window(win) -> Optional[_Window]:
    if win is None:
        return None
    nt, ny, nx, rt, ry, rx = (int(v) for v in win)
    return _Window(nt, ny, nx, rt, ry, rx)


# ------------------------------------------------------------------ mask stage

def pool_blocks(x: torch.Tensor, n_valid: Optional[int] = None, block: int = 64,
                blocks: Optional[Blocks] = None) -> torch.Tensor:
    B, H, N, d = _qkv(x, "x")
    n_valid = N if n_valid is None else n_valid
    nb = _nblocks(blocks, n_valid, block)
    out = torch.empty((B, H, nb, d), dtype=torch.float32, device=x.device)
    lib = load()
    bref = None if blocks is None else blocks._c()
    _check(lib.bsa_pool_blocks(x.data_ptr(), B, H, N, d, n_valid, block,
                               None if bref is None else ctypes.byref(bref), out.data_ptr(),
                               _stream(x.device)), "pool_blocks")
    return out


def select_blocks(qbar: torch.Tensor, kbar: torch.Tensor, thr: float, scale: float = 0.0,
                  q_sizes: Optional[torch.Tensor] = None, k_sizes: Optional[torch.Tensor] = None,
                  window=None, kv_stride: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    _dev_tensor(qbar, torch.float32, "qbar")
    _dev_tensor(kbar, torch.float32, "kbar")
    B, H, nqb, d = qbar.shape
    nkb = kbar.shape[2]
    kv_stride = nkb if kv_stride is None else kv_stride
    kv_count = torch.empty((B, H, nqb), dtype=torch.int32, device=qbar.device)
    kv_index = torch.full((B, H, nqb, kv_stride), -1, dtype=torch.int32, device=qbar.device)
    for t, n in ((q_sizes, "q_sizes"), (k_sizes, "k_sizes")):
        if t is not None:
            _dev_tensor(t, torch.int32, n)
    w = _window(window)
    lib = load()
    _check(lib.bsa_select_blocks(qbar.data_ptr(), kbar.data_ptr(), B, H, nqb, nkb, d, _ptr(q_sizes),
                                 _ptr(k_sizes), thr, scale, None if w is None else ctypes.byref(w),
                                 kv_count.data_ptr(), kv_index.data_ptr(), kv_stride,
                                 _stream(qbar.device)), "select_blocks")
    return kv_count, kv_index


def build_block_mask(q: torch.Tensor, k: torch.Tensor, thr: float, block: int = 64,
                     window=None, n_valid: Optional[int] = None, qb: Optional[Blocks] = None,
                     kb: Optional[Blocks] = None, kv_stride: Optional[int] = None,
                     out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                     workspace: Optional[torch.Tensor] = None):
    """Returns (kv_count [B,H,nqb] int32, kv_index [B,H,nqb,kv_stride] int32)."""
    B, H, N, d = _qkv(q, "q")
    if k.shape != q.shape:
        raise ValueError("q and k must have the same shape")
    _qkv(k, "k")
    n_valid = N if n_valid is None else n_valid
    nqb, nkb = _nblocks(qb, n_valid, block), _nblocks(kb, n_valid, block)
    kv_stride = nkb if kv_stride is None else kv_stride
    if out is None:
        kv_count = torch.empty((B, H, nqb), dtype=torch.int32, device=q.device)
        kv_index = torch.empty((B, H, nqb, kv_stride), dtype=torch.int32, device=q.device)
    else:
        kv_count, kv_index = out
    lib = load()
    ws_bytes = lib.bsa_build_block_mask_workspace(B, H, nqb, nkb, d)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    w = _window(window)
    qbc, kbc = (None if qb is None else qb._c()), (None if kb is None else kb._c())
    _check(lib.bsa_build_block_mask(q.data_ptr(), k.data_ptr(), B, H, N, d, n_valid, block,
                                    None if qbc is None else ctypes.byref(qbc),
                                    None if kbc is None else ctypes.byref(kbc), thr,
                                    None if w is None else ctypes.byref(w), kv_count.data_ptr(),
                                    kv_index.data_ptr(), kv_stride, workspace.data_ptr(), workspace.numel(),
                                    _stream(q.device)), "build_block_mask")
    return kv_count, kv_index


def build_centroid_mask(cq: torch.Tensor, q_sizes: torch.Tensor, ck: torch.Tensor,
                        k_sizes: torch.Tensor, top_p: float, scale: float = 0.0):
    _dev_tensor(cq, torch.float32, "cq")
    _dev_tensor(ck, torch.float32, "ck")
    _dev_tensor(q_sizes, torch.int32, "q_sizes")
    _dev_tensor(k_sizes, torch.int32, "k_sizes")
    B, H, Cq, d = cq.shape
    Ck = ck.shape[2]
    kv_count = torch.empty((B, H, Cq), dtype=torch.int32, device=cq.device)
    kv_index = torch.full((B, H, Cq, Ck), -1, dtype=torch.int32, device=cq.device)
    lib = load()
    _check(lib.bsa_build_centroid_mask(cq.data_ptr(), q_sizes.data_ptr(), ck.data_ptr(), k_sizes.data_ptr(),
                                       B, H, Cq, Ck, d, top_p, scale, kv_count.data_ptr(),
                                       kv_index.data_ptr(), Ck, _stream(cq.device)), "build_centroid_mask")
    return kv_count, kv_index


# ------------------------------------------------------------------ attention

def block_sparse_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_count: torch.Tensor,
                          kv_index: torch.Tensor, n_valid: Optional[int] = None, block: int = 64,
                          qb: Optional[Blocks] = None, kb: Optional[Blocks] = None, scale: float = 0.0,
                          out: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    B, H, N, d = _qkv(q, "q")
    for t, n in ((k, "k"), (v, "v")):
        if _qkv(t, n) != q.shape:
            raise ValueError(f"{n} must have the shape of q")
    _dev_tensor(kv_count, torch.int32, "kv_count")
    _dev_tensor(kv_index, torch.int32, "kv_index")
    n_valid = N if n_valid is None else n_valid
    nqb = _nblocks(qb, n_valid, block)
    if kv_count.numel() != B * H * nqb:
        raise ValueError("kv_count must have B*H*nqb entries")
    kv_stride = kv_index.shape[-1]
    if kv_index.numel() != B * H * nqb * kv_stride:
        raise ValueError("kv_index must be [B, H, nqb, kv_stride]")
    o = torch.empty_like(q) if out is None else out
    if out is not None:
        _qkv(o, "out")
    lib = load()
    qbc, kbc = (None if qb is None else qb._c()), (None if kb is None else kb._c())
    if workspace is None:
        ws_bytes = lib.bsa_block_sparse_attn_fwd_workspace(B, H, nqb, None if qbc is None else ctypes.byref(qbc))
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib.bsa_block_sparse_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, H, N, d,
                                         n_valid, block, None if qbc is None else ctypes.byref(qbc),
                                         None if kbc is None else ctypes.byref(kbc), kv_count.data_ptr(),
                                         kv_index.data_ptr(), kv_stride, scale,
                                         None if workspace is None else workspace.data_ptr(),
                                         0 if workspace is None else workspace.numel(),
                                         _stream(q.device)), "block_sparse_attn_fwd")
    return o


def block_sparse_attn_fwd_lse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_count: torch.Tensor,
                              kv_index: torch.Tensor, n_valid: Optional[int] = None, block: int = 64,
                              qb: Optional[Blocks] = None, kb: Optional[Blocks] = None, scale: float = 0.0,
                              out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                              workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The forward, plus each row's fp32 softmax log-normaliser [B, H, N]."""
    B, H, N, d = _qkv(q, "q")
    for t, n in ((k, "k"), (v, "v")):
        if _qkv(t, n) != q.shape:
            raise ValueError(f"{n} must have the shape of q")
    _dev_tensor(kv_count, torch.int32, "kv_count")
    _dev_tensor(kv_index, torch.int32, "kv_index")
    n_valid = N if n_valid is None else n_valid
    nqb = _nblocks(qb, n_valid, block)
    if kv_count.numel() != B * H * nqb:
        raise ValueError("kv_count must have B*H*nqb entries")
    kv_stride = kv_index.shape[-1]
    if kv_index.numel() != B * H * nqb * kv_stride:
        raise ValueError("kv_index must be [B, H, nqb, kv_stride]")
    o = torch.empty_like(q) if out is None else _dev_tensor(out, torch.bfloat16, "out")
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _dev_tensor(lse, torch.float32, "lse")
    if lse.numel() != B * H * N:
        raise ValueError("lse must have B*H*N entries")
    lib = load()
    qbc, kbc = (None if qb is None else qb._c()), (None if kb is None else kb._c())
    if workspace is None:
        ws_bytes = lib.bsa_block_sparse_attn_fwd_workspace(B, H, nqb, None if qbc is None else ctypes.byref(qbc))
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib.bsa_block_sparse_attn_fwd_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                             lse.data_ptr(), B, H, N, d, n_valid, block,
                                             None if qbc is None else ctypes.byref(qbc),
                                             None if kbc is None else ctypes.byref(kbc), kv_count.data_ptr(),
                                             kv_index.data_ptr(), kv_stride, scale,
                                             None if workspace is None else workspace.data_ptr(),
                                             0 if workspace is None else workspace.numel(),
                                             _stream(q.device)), "block_sparse_attn_fwd_lse")
    return o, lse


def block_sparse_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                          dout: torch.Tensor, lse: torch.Tensor, kv_count: torch.Tensor,
                          kv_index: torch.Tensor, n_valid: Optional[int] = None, block: int = 64,
                          scale: float = 0.0, out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                          workspace: Optional[torch.Tensor] = None, qb: Optional[Blocks] = None,
                          kb: Optional[Blocks] = None
                          ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Gradients (dq, dk, dv) of the block-sparse attention: uniform blocks, or
    descriptors (``qb``, ``kb``) bounded to 64 tokens (``max_len``)."""
    B, H, N, d = _qkv(q, "q")
    for t, n in ((k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        if _qkv(t, n) != q.shape:
            raise ValueError(f"{n} must have the shape of q")
    _dev_tensor(lse, torch.float32, "lse")
    if lse.numel() != B * H * N:
        raise ValueError("lse must have B*H*N entries")
    _dev_tensor(kv_count, torch.int32, "kv_count")
    _dev_tensor(kv_index, torch.int32, "kv_index")
    n_valid = N if n_valid is None else n_valid
    nqb = _nblocks(qb, n_valid, block)
    if kv_count.numel() != B * H * nqb:
        raise ValueError("kv_count must have B*H*nqb entries")
    kv_stride = kv_index.shape[-1]
    if kv_index.numel() != B * H * nqb * kv_stride:
        raise ValueError("kv_index must be [B, H, nqb, kv_stride]")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3)) if out is None else out
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        if _qkv(t, n) != q.shape:
            raise ValueError(f"{n} must have the shape of q")
    lib = load()
    qr, kr = _blocks_ref(qb), _blocks_ref(kb)
    ws_bytes = lib.bsa_block_sparse_attn_bwd_workspace(B, H, N, qr, kr)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    _check(lib.bsa_block_sparse_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                         lse.data_ptr(), B, H, N, d, n_valid, block, qr, kr, kv_count.data_ptr(),
                                         kv_index.data_ptr(), kv_stride, scale, dq.data_ptr(), dk.data_ptr(),
                                         dv.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                         _stream(q.device)), "block_sparse_attn_bwd")
    return dq, dk, dv


# ------------------------------------------------------------------ diagnostic

def attention_tile_stats(q: torch.Tensor, k: torch.Tensor, lse: torch.Tensor, n_valid: Optional[int] = None,
                         scale: float = 0.0):
    """Max, sum and min of the full attention per 64 x 64 tile: three fp32
    [B,H,nb,nb] tensors. ``lse`` [B,H,N] holds the full rows' normalisers."""
    B, H, N, d = _qkv(q, "q")
    n_valid = N if n_valid is None else n_valid
    _dev_tensor(lse, torch.float32, "lse")
    nb = -(-n_valid // 64)
    out = [torch.empty((B, H, nb, nb), dtype=torch.float32, device=q.device) for _ in range(3)]
    _check(load().bsa_attention_tile_stats(q.data_ptr(), k.data_ptr(), lse.data_ptr(), B, H, N, d, n_valid, scale,
                                           out[0].data_ptr(), out[1].data_ptr(), out[2].data_ptr(),
                                           _stream(q.device)), "attention_tile_stats")
    return tuple(out)


def mask_recall(tile_max: torch.Tensor, tile_sum: torch.Tensor, kv_count: torch.Tensor, kv_index: torch.Tensor):
    """Per query block: (oracle recall, mass recall) fp32 [B,H,nqb] each."""
    _dev_tensor(tile_max, torch.float32, "tile_max")
    _dev_tensor(tile_sum, torch.float32, "tile_sum")
    _dev_tensor(kv_count, torch.int32, "kv_count")
    _dev_tensor(kv_index, torch.int32, "kv_index")
    B, H, nqb, nkb = tile_max.shape
    rec = torch.empty((B, H, nqb), dtype=torch.float32, device=tile_max.device)
    mass = torch.empty_like(rec)
    _check(load().bsa_mask_recall(tile_max.data_ptr(), tile_sum.data_ptr(), kv_count.data_ptr(), kv_index.data_ptr(),
                                  kv_index.shape[-1], B, H, nqb, nkb, rec.data_ptr(), mass.data_ptr(),
                                  _stream(tile_max.device)), "mask_recall")
    return rec, mass


def check_mask(kv_count: torch.Tensor, kv_index: torch.Tensor, nkb: int):
    """Counts list defects: (rows with a count outside [0, kv_stride], ids
    outside [0, nkb), entries not greater than their predecessor)."""
    _dev_tensor(kv_count, torch.int32, "kv_count")
    _dev_tensor(kv_index, torch.int32, "kv_index")
    B, H, nqb, stride = kv_index.shape
    if kv_count.numel() != B * H * nqb:
        raise ValueError("kv_count must be [B, H, nqb]")
    bad = torch.empty(3, dtype=torch.int32, device=kv_index.device)
    _check(load().bsa_check_mask(kv_count.data_ptr(), kv_index.data_ptr(), B, H, nqb, nkb, stride, bad.data_ptr(),
                                 _stream(kv_index.device)), "check_mask")
    return tuple(int(v) for v in bad.cpu().tolist())


# ------------------------------------------------------------------ reorder

def _perm_args(x, perm):
    B, H, N, d = _qkv(x, "x")
    _dev_tensor(perm, torch.int32, "perm")
    if perm.numel() == N:
        per_head = 0
    elif perm.numel() == B * H * N:
        per_head = 1
    else:
        raise ValueError("perm must have N or B*H*N entries")
    return B, H, N, d, per_head


def permute_tokens(x: torch.Tensor, perm: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[b,h,i] = x[b,h,perm[i]]."""
    B, H, N, d, ph = _perm_args(x, perm)
    y = torch.empty_like(x) if out is None else out
    _check(load().bsa_permute_tokens(x.data_ptr(), y.data_ptr(), perm.data_ptr(), B, H, N, d, ph,
                                     _stream(x.device)), "permute_tokens")
    return y


def unpermute_tokens(x: torch.Tensor, perm: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[b,h,perm[i]] = x[b,h,i]."""
    B, H, N, d, ph = _perm_args(x, perm)
    y = torch.empty_like(x) if out is None else out
    _check(load().bsa_unpermute_tokens(x.data_ptr(), y.data_ptr(), perm.data_ptr(), B, H, N, d, ph,
                                       _stream(x.device)), "unpermute_tokens")
    return y


def fractal_order(T: int, Hl: int, Wl: int, P: int, N: Optional[int] = None):
    """Host function. Returns int32 CPU tensors (perm [N], start [nb], length [nb], coords [nb, 3])."""
    n = T * Hl * Wl
    N = n if N is None else N
    nb_max = T * (-(-Hl // P)) * (-(-Wl // P))
    perm = torch.empty(N, dtype=torch.int32)
    st = torch.empty(nb_max, dtype=torch.int32)
    ln = torch.empty(nb_max, dtype=torch.int32)
    co = torch.empty((nb_max, 3), dtype=torch.int32)
    nb = ctypes.c_int(0)
    _check(load().bsa_fractal_order(T, Hl, Wl, P, N, perm.data_ptr(), st.data_ptr(), ln.data_ptr(),
                                    co.data_ptr(), nb_max, ctypes.byref(nb)), "fractal_order")
    return perm, st[:nb.value], ln[:nb.value], co[:nb.value]


def tile_order(T: int, Hl: int, Wl: int, pt: int, ph: int, pw: int, N: Optional[int] = None):
    """Host function: pt x ph x pw boxes as contiguous blocks. Returns int32 CPU
    tensors (perm [N], start [nb], length [nb], coords [nb, 3])."""
    n = T * Hl * Wl
    N = n if N is None else N
    nb_max = (-(-T // pt)) * (-(-Hl // ph)) * (-(-Wl // pw)) if min(pt, ph, pw) > 0 else 1
    perm = torch.empty(N, dtype=torch.int32)
    st = torch.empty(nb_max, dtype=torch.int32)
    ln = torch.empty(nb_max, dtype=torch.int32)
    co = torch.empty((nb_max, 3), dtype=torch.int32)
    nb = ctypes.c_int(0)
    _check(load().bsa_tile_order(T, Hl, Wl, pt, ph, pw, N, perm.data_ptr(), st.data_ptr(), ln.data_ptr(),
                                 co.data_ptr(), nb_max, ctypes.byref(nb)), "tile_order")
    return perm, st[:nb.value], ln[:nb.value], co[:nb.value]


# ------------------------------------------------------------------ clustering

def kmeans(x: torch.Tensor, C: int, iters: int, uniforms: torch.Tensor, n_valid: Optional[int] = None):
    """Returns (centroids [B,H,C,d] fp32, assign [B,H,N] int32, sizes [B,H,C] int32)."""
    B, H, N, d = _qkv(x, "x")
    n_valid = N if n_valid is None else n_valid
    _dev_tensor(uniforms, torch.float32, "uniforms")
    if uniforms.numel() != B * H * C:
        raise ValueError("uniforms must be [B, H, C]")
    cent = torch.empty((B, H, C, d), dtype=torch.float32, device=x.device)
    assign = torch.empty((B, H, N), dtype=torch.int32, device=x.device)
    sizes = torch.empty((B, H, C), dtype=torch.int32, device=x.device)
    lib = load()
    ws_bytes = lib.bsa_kmeans_workspace(B, H, N, C, d)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    _check(lib.bsa_kmeans(x.data_ptr(), B, H, N, d, n_valid, C, iters, uniforms.data_ptr(), cent.data_ptr(),
                          assign.data_ptr(), sizes.data_ptr(), ws.data_ptr(), ws.numel(), _stream(x.device)),
           "kmeans")
    return cent, assign, sizes


def kmeans_warm(x: torch.Tensor, centroids: torch.Tensor, max_iters: int, n_valid: Optional[int] = None,
                tol_moves: int = 0):
    """Lloyd rounds from the given centroids [B,H,C,d] (not modified), stopping
    per head after the first round that moves at most tol_moves tokens.
    Returns (centroids, assign, sizes, changes [B,H,max_iters])."""
    B, H, N, d = _qkv(x, "x")
    n_valid = N if n_valid is None else n_valid
    _dev_tensor(centroids, torch.float32, "centroids")
    if centroids.dim() != 4 or centroids.shape[:2] != (B, H) or centroids.shape[3] != d:
        raise ValueError("centroids must be [B, H, C, d]")
    C = centroids.shape[2]
    cent = centroids.clone()
    assign = torch.empty((B, H, N), dtype=torch.int32, device=x.device)
    sizes = torch.empty((B, H, C), dtype=torch.int32, device=x.device)
    changes = torch.empty((B, H, max(max_iters, 1)), dtype=torch.int32, device=x.device)
    lib = load()
    ws_bytes = lib.bsa_kmeans_workspace(B, H, N, C, d)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    _check(lib.bsa_kmeans_warm(x.data_ptr(), B, H, N, d, n_valid, C, max_iters, tol_moves, cent.data_ptr(),
                               assign.data_ptr(),
                               sizes.data_ptr(), changes.data_ptr(), ws.data_ptr(), ws.numel(), _stream(x.device)),
           "kmeans_warm")
    return cent, assign, sizes, changes


def cluster_order(assign: torch.Tensor, C: int, n_valid: Optional[int] = None):
    """Returns (perm [B,H,N], start [B,H,C], length [B,H,C]) int32."""
    _dev_tensor(assign, torch.int32, "assign")
    B, H, N = assign.shape
    n_valid = N if n_valid is None else n_valid
    perm = torch.empty((B, H, N), dtype=torch.int32, device=assign.device)
    start = torch.empty((B, H, C), dtype=torch.int32, device=assign.device)
    length = torch.empty((B, H, C), dtype=torch.int32, device=assign.device)
    lib = load()
    ws_bytes = lib.bsa_cluster_order_workspace(B, H, N, C)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=assign.device)
    _check(lib.bsa_cluster_order(assign.data_ptr(), B, H, N, n_valid, C, perm.data_ptr(), start.data_ptr(),
                                 length.data_ptr(), ws.data_ptr(), ws.numel(), _stream(assign.device)),
           "cluster_order")
    return perm, start, length
