"""Composed hot paths built from the C-ABI calls (argument marshalling only).

``fractal_sta_attention`` -- NABLA summary, Metodologia sections 1-3: tokens
are reordered by fractal flattening, the content-adaptive CDF mask is built
on the patch blocks and OR'd with the static sliding-tile window, attention
runs over the kept patch tiles and the output is put back in raster order.

``head_tiled_attention`` -- Veda summary, section 2.2: every head has its
own p_t x p_h x p_w factorisation of the tile, so each head gets its own token
order and its own box blocks; the CDF mask and the attention then run over
each head's boxes and the output returns to raster order.

``mask_quality`` -- Veda summary, sections 2.1 and 3: the full attention is
max-pooled (and summed, min-pooled) over every 64 x 64 tile in two passes
(row normalisers from the forward with every block kept, then the tile map),
and a block mask is scored by its recall against the max-pooled oracle mask
of the same budget and by the attention mass it keeps.

``semantic_attention`` -- Sparse VideoGen2 summary, Metodologia A-C: Q and K
are clustered with k-means, tokens are permuted cluster-contiguously, the
centroid top-p rule selects key clusters per query cluster, attention runs
over the variable-size cluster blocks and the output is inverse-permuted.

Every arithmetic step runs in libbsa's HIP kernels; this module only chains
the calls and keeps the intermediate tensors.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import torch

from . import (Blocks, attention_tile_stats, block_sparse_attn_fwd, block_sparse_attn_fwd_lse,
               build_block_mask, build_centroid_mask, cluster_order, fractal_order, kmeans, mask_recall,
               permute_tokens, tile_order, unpermute_tokens)


@dataclasses.dataclass
class FractalLayout:
    """Fractal order of a T x Hl x Wl latent video with P x P patches, on the device."""
    perm: torch.Tensor          # int32 [N]
    blocks: Blocks              # one block per patch
    grid: Tuple[int, int, int]  # (T, ceil(Hl/P), ceil(Wl/P)) block grid
    coords: torch.Tensor        # int32 [nblocks, 3] (host)


def fractal_layout(T: int, Hl: int, Wl: int, P: int, N: int, device, bound_blocks: bool = True) -> FractalLayout:
    """``bound_blocks``: pass the longest patch as the blocks' length bound
    (when it is at most 64), so attention takes each patch as one tile."""
    perm, st, ln, co = fractal_order(T, Hl, Wl, P, N)
    grid = (T, -(-Hl // P), -(-Wl // P))
    mx = int(ln.max()) if bound_blocks and len(ln) else 0
    return FractalLayout(perm.to(device), Blocks(st.to(device), ln.to(device), mx if mx <= 64 else 0), grid, co)


def fractal_sta_attention(q, k, v, layout: FractalLayout, thr: float,
                          radius: Optional[Tuple[int, int, int]] = (1, 2, 2),
                          n_valid: Optional[int] = None, return_mask: bool = False):
    """Reorder -> CDF mask (OR window) -> block-sparse attention -> inverse reorder."""
    qp = permute_tokens(q, layout.perm)
    kp = permute_tokens(k, layout.perm)
    vp = permute_tokens(v, layout.perm)
    window = None if radius is None else (*layout.grid, *radius)
    cnt, idx = build_block_mask(qp, kp, thr, window=window, n_valid=n_valid,
                                qb=layout.blocks, kb=layout.blocks)
    op = block_sparse_attn_fwd(qp, kp, vp, cnt, idx, n_valid=n_valid,
                               qb=layout.blocks, kb=layout.blocks)
    o = unpermute_tokens(op, layout.perm)
    return (o, cnt, idx) if return_mask else o


@dataclasses.dataclass
class HeadTiling:
    """Per-head box orders of a T x Hl x Wl latent, on the device."""
    perm: torch.Tensor          # int32 [B, H, N]: head h's token order
    blocks: Blocks              # per head [B, H, nb]: head h's boxes, then empty blocks
    factors: Tuple[Tuple[int, int, int], ...]   # (pt, ph, pw) of each head
    nblocks: Tuple[int, ...]    # real boxes of each head


def head_tiling_layout(T: int, Hl: int, Wl: int, factors, N: int, B: int, device,
                       bound_blocks: bool = True) -> HeadTiling:
    """One ``tile_order`` per head; block lists are padded to a common count
    with blocks of length 0 (they take no part in the mask). ``bound_blocks``
    passes the longest box (when at most 64 tokens) as the length bound."""
    orders = [tile_order(T, Hl, Wl, *f, N) for f in factors]
    nb = max(len(o[1]) for o in orders)
    H = len(factors)
    perm = torch.stack([o[0] for o in orders])
    st = torch.full((H, nb), T * Hl * Wl, dtype=torch.int32)
    ln = torch.zeros((H, nb), dtype=torch.int32)
    for h, o in enumerate(orders):
        st[h, :len(o[1])] = o[1]
        ln[h, :len(o[2])] = o[2]

    def dev(x):
        return x.unsqueeze(0).expand(B, *x.shape).contiguous().to(device)
    mx = int(ln.max()) if bound_blocks else 0
    return HeadTiling(dev(perm), Blocks(dev(st), dev(ln), mx if mx <= 64 else 0), tuple(tuple(f) for f in factors),
                      tuple(len(o[1]) for o in orders))


def head_tiled_attention(q, k, v, layout: HeadTiling, thr: float, n_valid: Optional[int] = None,
                         return_mask: bool = False):
    """Per-head reorder -> CDF mask over each head's boxes -> attention -> inverse reorder."""
    qp = permute_tokens(q, layout.perm)
    kp = permute_tokens(k, layout.perm)
    vp = permute_tokens(v, layout.perm)
    cnt, idx = build_block_mask(qp, kp, thr, n_valid=n_valid, qb=layout.blocks, kb=layout.blocks)
    op = block_sparse_attn_fwd(qp, kp, vp, cnt, idx, n_valid=n_valid, qb=layout.blocks, kb=layout.blocks)
    o = unpermute_tokens(op, layout.perm)
    return (o, cnt, idx) if return_mask else o


@dataclasses.dataclass
class MaskQuality:
    """Full-attention tile map and the recall of one mask against it (device)."""
    tile_max: torch.Tensor       # fp32 [B,H,nb,nb]
    tile_sum: torch.Tensor
    tile_min: torch.Tensor
    oracle_recall: torch.Tensor  # fp32 [B,H,nb]
    mass_recall: torch.Tensor


def mask_quality(q, k, kv_count, kv_index, n_valid: Optional[int] = None) -> MaskQuality:
    """Two passes over the full attention of (q, k), then the mask's recall."""
    B, H, N, _ = q.shape
    n_valid = N if n_valid is None else n_valid
    nb = -(-n_valid // 64)
    full_c = torch.full((B, H, nb), nb, dtype=torch.int32, device=q.device)
    full_i = torch.arange(nb, dtype=torch.int32, device=q.device).expand(B, H, nb, nb).contiguous()
    _, lse = block_sparse_attn_fwd_lse(q, k, k, full_c, full_i, n_valid=n_valid)   # only lse is used
    tmax, tsum, tmin = attention_tile_stats(q, k, lse, n_valid)
    rec, mass = mask_recall(tmax, tsum, kv_count, kv_index)
    return MaskQuality(tmax, tsum, tmin, rec, mass)


@dataclasses.dataclass
class SemanticState:
    """Intermediate results of the semantic path (all on the device)."""
    cq: torch.Tensor
    nq: torch.Tensor
    ck: torch.Tensor
    nk: torch.Tensor
    perm_q: torch.Tensor
    perm_k: torch.Tensor
    qblocks: Blocks
    kblocks: Blocks
    kv_count: torch.Tensor
    kv_index: torch.Tensor


def semantic_attention(q, k, v, Cq: int, Ck: int, iters: int, top_p: float,
                       uq: torch.Tensor, uk: torch.Tensor, n_valid: Optional[int] = None,
                       return_state: bool = False):
    """k-means(Q), k-means(K) -> cluster order -> centroid top-p -> attention -> inverse."""
    N = q.shape[2]
    n_valid = N if n_valid is None else n_valid
    cq, aq, nq = kmeans(q, Cq, iters, uq, n_valid)
    ck, ak, nk = kmeans(k, Ck, iters, uk, n_valid)
    pq, sq, lq = cluster_order(aq, Cq, n_valid)
    pk, sk, lk = cluster_order(ak, Ck, n_valid)
    qp = permute_tokens(q, pq)
    kp = permute_tokens(k, pk)
    vp = permute_tokens(v, pk)
    cnt, idx = build_centroid_mask(cq, nq, ck, nk, top_p)
    qb, kb = Blocks(sq, lq), Blocks(sk, lk)
    op = block_sparse_attn_fwd(qp, kp, vp, cnt, idx, n_valid=n_valid, qb=qb, kb=kb)
    o = unpermute_tokens(op, pq)
    if return_state:
        return o, SemanticState(cq, nq, ck, nk, pq, pk, qb, kb, cnt, idx)
    return o
